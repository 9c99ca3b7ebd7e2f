"""GPU parity of the group size 32 format (one fp32 scale, and zero point, per 32 rows of a
column; P3 lists g among the format choices) through the dense decode and prefill kernels.
A 128-deep superblock holds four groups: the prefill kernel closes a group after every
32-deep MFMA step; the decode kernels run each 64-deep MFMA twice, once per group, with the
other group's lanes of the weight operand zeroed.

Same gates as the other formats: INT32 per-group partials bit for bit against the oracle,
float outputs through gpu_cases.check_float_output, w4a8_linear bit-identical to quant_act
followed by gemm."""
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


def _prep(M, K, N, asym, bits, seed):
    Xb = W.random_activations(seed, M, K, outlier_cols=2, outlier_scale=20.0)
    Wt = W.random_weights(seed + 1, K, N)
    Wt[:32, 0] = 0.0                                    # an all-zero group
    d = L.desc(K, N, 32, asym, bits=bits)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    codes, scales, zeros = O.quant_weight(Wt, 32, asym, bits)
    return Xb, d, blob, codes, scales, zeros


@pytest.mark.parametrize("M,K,N,asym,bits", [
    (1, 4096, 256, False, 4),      # decode, one chunk
    (8, 1024, 96, True, 4),
    (32, 4096, 512, True, 4),      # 32-row tile
    (32, 8192, 64, False, 4),      # several chunks
    (12, 14336, 48, True, 4),      # long K: 8 slices
    (16, 2048, 80, False, 8),      # 8-bit codes
    (300, 1024, 272, True, 4),     # prefill kernel
    (257, 512, 129, False, 4),
    (64, 768, 256, False, 8),
])
def test_g32_partials_bit_exact(M, K, N, asym, bits):
    _print(f"g32 partials M={M} K={K} N={N} asym={asym} bits={bits}")
    Xb, d, blob, codes, scales, zeros = _prep(M, K, N, asym, bits, M * 13 + K + N)
    assert L.w4a8_kernel_name(d, M).endswith("_g32")
    Xq, _ = gpu_quant(Xb)
    P = torch.full((M, N, K // 32), -7, dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, _ = O.quant_act(W.bf16_values(Xb))
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, zeros, 32))


@pytest.mark.parametrize("M,K,N,asym,bits", [(1, 4096, 14336, False, 4), (32, 4096, 14336, True, 4),
                                             (300, 1024, 272, True, 4), (1000, 512, 1000, False, 4),
                                             (33, 2048, 64, False, 8), (8, 4096, 512, False, 8)])
def test_g32_gemm_outputs(M, K, N, asym, bits):
    Xb, d, blob, codes, scales, zeros = _prep(M, K, N, asym, bits, M * 5 + N + K)
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    Y64 = O.gemm(q, s, codes, scales, zeros, 32)
    _print(check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), Y64))


@pytest.mark.parametrize("M,K,N,asym,bits", [(1, 4096, 1024, True, 4), (2, 4096, 512, False, 4),
                                             (16, 512, 72, True, 4), (1, 8192, 80, False, 8),
                                             (8, 4096, 256, True, 4)])
def test_g32_linear_matches_quant_then_gemm(M, K, N, asym, bits):
    Xb, d, blob, _, _, _ = _prep(M, K, N, asym, bits, M * 3 + K + 2 * N)
    X = Xb.to(DEV)
    for dt, tdt in ((L.W4A8_OUT_F32, torch.float32), (L.W4A8_OUT_BF16, torch.bfloat16)):
        Xq1, sx1 = gpu_quant(Xb)
        Y1 = torch.empty((M, N), dtype=tdt, device=DEV)
        L.w4a8_gemm(Xq1, sx1, blob, d, Y1, dt)
        Xq2 = torch.full((M, K), 99, dtype=torch.int8, device=DEV)
        sx2 = torch.full((M,), -1.0, dtype=torch.float32, device=DEV)
        Y2 = torch.empty((M, N), dtype=tdt, device=DEV)
        L.w4a8_linear(X, blob, d, Y2, Xq2, sx2, dt)
        assert torch.equal(Xq1, Xq2)
        iv = torch.int16 if tdt == torch.bfloat16 else torch.int32
        assert torch.equal(Y1.view(iv), Y2.view(iv))
