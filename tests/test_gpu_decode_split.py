"""GPU parity of the dense decode GEMM with one K-slice per wave (4-bit codes, g in {64, 128},
up to 32 rows in 16- or 32-row tiles, 2048 < K <= 4096; P1 section 5.2, P5 section 7).

Each case runs w4a8_gemm through the C-ABI and checks the float32 and bfloat16 outputs against the
oracle (gpu_cases.check_float_output: float32 within 1e-3 of the float64 product, bfloat16 equal to
the round-to-nearest-even of the float32 output).  The shapes reach the kernel's edges: ragged N
(a workgroup's last column tiles past N), ragged K (waves whose slice is partly or wholly past K),
row counts that leave part of the 16- or 32-row tile empty, asymmetric codes, binary16 scales, and a
strided output whose columns past N must stay untouched."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, check_float_output, device_blob, gpu_quant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("M,K,N,g,asym,h16", [
    (17, 4096, 40, 128, False, False),    # 3 of 4 tile slots, 17 of 32 rows
    (17, 2176, 72, 64, True, False),      # 17 superblocks: wave 8 has one, waves 9-15 none
    (31, 3072, 1024, 128, True, False),   # 24 superblocks, 31 of 32 rows
    (32, 4096, 96, 64, False, False),
    (24, 2560, 48, 128, False, True),     # binary16 scales
    (20, 4096, 64, 64, True, True),
    (32, 4096, 14336, 128, False, False),  # the decode projection at 32 rows
    (18, 3968, 200, 128, True, False),    # 31 superblocks, ragged N inside a tile
    # 16-row tiles (rows that w4a8_linear does not quantize inside the chunked kernel)
    (3, 4096, 40, 128, False, False),     # 3 of 4 tile slots, 3 of 16 rows
    (8, 4096, 14336, 128, False, False),  # the decode projection at 8 rows
    (16, 3072, 1024, 64, True, False),
    (4, 2176, 72, 128, True, False),      # 17 superblocks
    (9, 2560, 48, 64, False, True),       # binary16 scales
    (11, 3968, 200, 128, False, False),
])
def test_decode_split_vs_oracle(M, K, N, g, asym, h16):
    _print(f"decode split M={M} K={K} N={N} g={g} asym={asym} h16={h16}")
    Xb = W.random_activations(M * 13 + K + N, M, K, outlier_cols=3, outlier_scale=30.0)
    x = W.bf16_values(Xb)
    x[2] = 0.0                                          # an all-zero row: scale 0, outputs 0
    Xb = W.to_bf16(x)
    Wt = W.random_weights(K * 3 + N, K, N)
    Wt[:g, 0] = 0.0                                     # an all-zero group
    d = L.desc(K, N, g, asym, scale_bits=16 if h16 else 32)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    ldy = N + 24
    y32 = torch.full((M, ldy), 7.0, dtype=torch.float32, device=DEV)
    ybf = torch.full((M, ldy), 7.0, dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32[:, :N], L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf[:, :N], L.W4A8_OUT_BF16)
    assert torch.all(y32[:, N:] == 7.0) and torch.all(ybf[:, N:] == 7.0)
    q, s = O.quant_act(x)
    codes, scales, zeros = O.quant_weight(Wt, g, asym, scale_bits=16 if h16 else 32)
    Y64 = O.gemm(q, s, codes, scales, zeros, g)
    assert np.all(y32[2, :N].cpu().numpy() == 0.0)
    _print(check_float_output(y32[:, :N].cpu().numpy(), ybf[:, :N].float().cpu().numpy(), Y64))


def test_decode_split_run_twice_identical():
    """Two calls give the same bits (the slice sums are added in a fixed order)."""
    M, K, N = 32, 4096, 2048
    Xb = W.random_activations(77, M, K, outlier_cols=2, outlier_scale=50.0)
    Wt = W.random_weights(78, K, N)
    d = L.desc(K, N, 128, False)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    ys = []
    for _ in range(2):
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        L.w4a8_gemm(Xq, sx, blob, d, y, L.W4A8_OUT_F32)
        ys.append(y.view(torch.int32).clone())
    assert torch.equal(ys[0], ys[1])

