"""GPU parity of the W4A16 sibling (bfloat16 activations, the 4-bit codes of the W4A8 blob
dequantized in the kernel) against the oracle's gemm_a16, through the C-ABI, with the float
gates of the W4A8 GEMM: float32 mode within 1e-3 of the float64 oracle, bfloat16 mode equal to
the round-to-nearest-even of the float32 mode, and within one bfloat16 step of the correctly
rounded oracle."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, check_float_output, device_blob

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _case(M, K, N, g, asym, seed, outliers=2, oscale=30.0, codes=False):
    Xb = W.random_activations(seed, M, K, outlier_cols=outliers, outlier_scale=oscale)
    d = L.desc(K, N, g, asym)
    if codes:
        c = W.random_codes(seed + 1, K, N, g, asym)
        blob = device_blob(d, L.w4a8_pack_codes(d, *c))
        cq, sc, z = c
    else:
        Wt = W.random_weights(seed + 2, K, N)
        blob = device_blob(d, L.w4a8_pack(d, Wt))
        cq, sc, z = O.quant_weight(Wt, g, asym)
    X = Xb.to(DEV)
    y32 = torch.full((M, N), 5.0, dtype=torch.float32, device=DEV)
    ybf = torch.full((M, N), 5.0, dtype=torch.bfloat16, device=DEV)
    L.w4a16_gemm(X, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a16_gemm(X, blob, d, ybf, L.W4A8_OUT_BF16)
    Y64 = O.gemm_a16(W.bf16_values(Xb), cq, sc, z, g)
    return check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), Y64)


@pytest.mark.parametrize("M,K,N,g,asym", [(1, 4096, 14336, 128, False), (8, 4096, 14336, 128, False),
                                          (32, 4096, 14336, 128, False), (16, 1024, 1024, 128, False),
                                          (5, 512, 40, 64, True), (3, 384, 33, 128, True), (17, 7168, 96, 64, True),
                                          (32, 8192, 48, 128, True), (2, 128, 16, 64, False), (20, 14336, 64, 128, True),
                                          # 16-row tiles over several 16-superblock chunks, the last one ragged
                                          (4, 2176, 72, 64, True), (12, 7168, 200, 128, False), (16, 3200, 64, 64, False)])
def test_w4a16_decode_vs_oracle(M, K, N, g, asym):
    """Decode shapes (M <= 32): 16- and 32-row tiles, one and several K chunks, ragged N, a K of
    one superblock, symmetric and asymmetric codes, g = 64 and 128."""
    _print(f"w4a16 M={M} K={K} N={N} g={g} asym={asym}", _case(M, K, N, g, asym, M + K + N))


def test_w4a16_full_code_range_and_zero_rows():
    """Random codes over the whole code range (every nibble, zero points 4..11), a zero row and a
    row of large values."""
    M, K, N, g = 9, 1024, 64, 64
    Xb = W.random_activations(3, M, K)
    x = W.bf16_values(Xb)
    x[2] = 0.0
    x[5] *= 1000.0
    Xb = W.to_bf16(x)
    for asym in (False, True):
        d = L.desc(K, N, g, asym)
        c = W.random_codes(11, K, N, g, asym)
        blob = device_blob(d, L.w4a8_pack_codes(d, *c))
        y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
        ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        L.w4a16_gemm(Xb.to(DEV), blob, d, y32, L.W4A8_OUT_F32)
        L.w4a16_gemm(Xb.to(DEV), blob, d, ybf, L.W4A8_OUT_BF16)
        Y64 = O.gemm_a16(W.bf16_values(Xb), *c, g)
        _print(check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), Y64))
        assert not y32[2].any()


def test_w4a16_strided_activations_and_output():
    """Row strides of X and Y larger than K and N."""
    M, K, N, g = 7, 512, 48, 128
    Xb = W.random_activations(21, M, K + 64)
    d = L.desc(K, N, g, True)
    Wt = W.random_weights(22, K, N)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    X = Xb.to(DEV)[:, :K]
    big = torch.zeros((M, N + 16), dtype=torch.float32, device=DEV)
    L.w4a16_gemm(X, blob, d, big[:, :N], L.W4A8_OUT_F32)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a16_gemm(X, blob, d, ybf, L.W4A8_OUT_BF16)
    cq, sc, z = O.quant_weight(Wt, g, True)
    Y64 = O.gemm_a16(W.bf16_values(Xb)[:, :K], cq, sc, z, g)
    _print(check_float_output(big[:, :N].cpu().numpy(), ybf.float().cpu().numpy(), Y64))
    assert not big[:, N:].any()


@pytest.mark.parametrize("M,K,N,g,asym", [(33, 512, 96, 128, True), (100, 1024, 200, 64, False),
                                          (128, 128, 128, 128, False), (257, 384, 129, 64, True),
                                          (300, 4096, 64, 128, True), (64, 2048, 1000, 64, False)])
def test_w4a16_prefill_vs_oracle(M, K, N, g, asym):
    """Prefill shapes (M > 32): 128 x 128 tiles with ragged rows and columns, one and many
    superblocks, both group sizes, symmetric and asymmetric codes."""
    assert L.w4a16_kernel_name(L.desc(K, N, g, asym), M).startswith("w4a16_prefill")
    _print(f"w4a16 prefill M={M} K={K} N={N} g={g} asym={asym}", _case(M, K, N, g, asym, 3 * M + K + N))


def test_w4a16_prefill_full_size_sampled_rows():
    """The up projection at full size (M = 4096, K = 4096, N = 14336, asymmetric g128) in the
    benchmark's launch configuration; the oracle checks 24 sampled rows (every column)."""
    cfg = W.C3_UP
    Xb, Wt = W.dense_inputs(cfg)
    d = L.desc(cfg.K, cfg.N, cfg.group_size, cfg.asymmetric)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    X = Xb.to(DEV)
    y32 = torch.empty((cfg.M, cfg.N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=DEV)
    L.w4a16_gemm(X, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a16_gemm(X, blob, d, ybf, L.W4A8_OUT_BF16)
    rows = np.sort(np.random.default_rng(7).choice(cfg.M, 24, replace=False))
    rows[0], rows[-1] = 0, cfg.M - 1
    cq, sc, z = O.quant_weight(Wt, cfg.group_size, cfg.asymmetric)
    Y64 = O.gemm_a16(W.bf16_values(Xb)[rows], cq, sc, z, cfg.group_size)
    _print(check_float_output(y32.cpu().numpy()[rows], ybf.float().cpu().numpy()[rows], Y64))
