"""GPU parity of the prefill GEMM's float outputs for small groups (g = 64 and g = 32; P3 lists g
among the format choices): two and four group epilogues per superblock, which set the prefill
kernel's register budget (each 32-deep MFMA step closes a group at g = 32, every second one at
g = 64).

Gates: float outputs through gpu_cases.check_float_output against the float64 oracle, on ragged
shapes (M and N not multiples of the 128 x 128 tile, N not a multiple of 16, one superblock, an
odd number of superblocks), both zero-point forms and both scale widths (binary16 scales at
g = 64 only: the format defines them for g in {64, 128}); and the C3 up
projection's shape at full size (the benchmark's launch configuration), on sampled rows."""
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


def _run(Xb, Wt, g, asym, sbits, rows=None):
    M, K = Xb.shape
    N = Wt.shape[1]
    d = L.desc(K, N, g, asym, scale_bits=sbits)
    assert L.w4a8_kernel_name(d, M).startswith("w4a8_prefill")
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    q, s = O.quant_act(W.bf16_values(Xb)[rows])
    assert np.array_equal(Xq.cpu().numpy()[rows], q)
    codes, scales, zeros = O.quant_weight(Wt, g, asym, scale_bits=sbits)
    Y64 = O.gemm(q, s, codes, scales, zeros, g)
    return check_float_output(y32.cpu().numpy()[rows], ybf.float().cpu().numpy()[rows], Y64)


@pytest.mark.parametrize("M,K,N,g,asym,sbits", [
    (33, 128, 64, 64, True, 32),       # smallest prefill M, one superblock
    (129, 512, 136, 64, True, 32),     # a one-row second M tile, N ends mid 16-column tile
    (257, 384, 129, 32, False, 32),    # odd superblock count, one column past a tile
    (300, 1024, 272, 32, True, 32),
    (1000, 256, 1000, 64, False, 16),  # binary16 scales
    (64, 2048, 520, 32, True, 32),
    (200, 640, 392, 64, True, 16),
    (512, 4096, 256, 64, True, 16),
])
def test_small_group_prefill_outputs(M, K, N, g, asym, sbits):
    _print(f"small-group prefill M={M} K={K} N={N} g={g} asym={asym} scale_bits={sbits}")
    Xb = W.random_activations(M * 7 + K + N + g, M, K, outlier_cols=2, outlier_scale=25.0)
    rs = np.random.default_rng(M + N)
    Wt = (W.random_weights(K * 5 + N + g, K, N) * rs.uniform(1e-2, 10, (1, N))).astype(np.float32)
    Wt[:g, 0] = 0.0                                     # an all-zero group
    Wt[g:2 * g, N - 1] = 0.0
    _print(_run(Xb, Wt, g, asym, sbits))


@pytest.mark.parametrize("g", [64, 32])
def test_small_group_prefill_full_size_sampled_rows(g):
    """The up projection (M = 4096, K = 4096, N = 14336, asymmetric) at g = 64 and g = 32 in the
    benchmark's launch configuration; the oracle checks 32 sampled rows (every column)."""
    cfg = W.C3_UP
    _print(f"small-group prefill full size g={g}")
    Xb, Wt = W.dense_inputs(cfg)
    rows = np.sort(np.random.default_rng(cfg.seed + g).choice(cfg.M, 32, replace=False))
    rows[0], rows[-1] = 0, cfg.M - 1
    _print(_run(Xb, Wt, g, cfg.asymmetric, 32, rows))
