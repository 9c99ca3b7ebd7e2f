"""GPU parity of the grouped gate/up GEMM with the static SiLU-requant folded into its epilogue
(w4a8_moe_gemm_silu_static; P1 section 8: act-quant folded into the GEMM; section 3.2: static
per-expert scales).

Two gates per case:
  1. bit for bit equal to the unfused chain w4a8_moe_gemm -> w4a8_silu_mul_quant_static on the
     same inputs (codes and row scales), on every row an expert owns;
  2. against the oracle's SiLU-requant (oracle.silu_mul, oracle.quant_act_static) of the chain's
     bf16 gate/up output: codes equal except within SILU_TIE_WINDOW of a rounding tie (the GPU's
     expf and numpy's exp differ by ulps), and the row scales equal.
The grouped GEMM itself is pinned against the oracle in test_gpu_parity.py.  The cases reach
every kernel that serves a grouped launch: the streaming kernel (K <= 4096, 16- and 32-row
tiles), the 128-row MFMA tiles of experts with many rows, the K-slice kernel (4096 < K <= 8192,
16-row tiles) and the chunked decode kernel (32-row tiles past K = 4096, and K > 8192)."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, SILU_TIE_WINDOW, gpu_quant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _fused_vs_chain(T, E, k, K, I, g, asym, seed, gather, zipf=0.0, bad_scales=False):
    cfg = W.MoEConfig("fz", T, K, I, E, k, g, asym, seed, zipf_s=zipf)
    ids, _ = W.moe_routing(cfg)
    R = T * k
    d = L.desc(K, 2 * I, g, asym)
    touched = sorted(set(ids.ravel().tolist()))
    host = {e: L.w4a8_pack_codes(d, *W.random_codes(seed * 31 + e, K, 2 * I, g, asym)) for e in touched}
    dev = L.experts_to_device(d, E, host)
    Xb = W.random_activations(seed, T, K, outlier_cols=2, outlier_scale=25.0)
    Xq, sx = gpu_quant(Xb)
    rows = torch.empty(R, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    if not gather:
        # rows already in sorted order: gather them on the host side of the test
        Xq = Xq[rows.long() // k].contiguous()
        sx = sx[rows.long() // k].contiguous()
    gth = rows if gather else None
    # chain: bf16 gate/up, then the static SiLU-requant
    GU = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, gth, k, off, E, R, dev.blob, dev.stride, d, GU)
    gu_np = W.bf16_values(GU.cpu())
    h = O.silu_mul(gu_np)
    rs = np.random.default_rng(seed)
    s_e = np.zeros(E, np.float32)
    offs = off.cpu().numpy()
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a < b:
            s_e[e] = np.float32(np.max(np.abs(h[a:b])) / 127 * rs.uniform(0.5, 1.3))
    if bad_scales:
        s_e[touched[0]] = 0.0
        s_e[touched[-1]] = np.inf
    s_d = torch.from_numpy(s_e).to(DEV)
    Hq1 = torch.full((R, I), 99, dtype=torch.int8, device=DEV)
    sh1 = torch.full((R,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_silu_mul_quant_static(GU, off, E, s_d, Hq1, sh1)
    # fused
    Hq2 = torch.full((R, I), 99, dtype=torch.int8, device=DEV)
    sh2 = torch.full((R,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_moe_gemm_silu_static(Xq, sx, gth, k, off, E, R, dev.blob, dev.stride, d, s_d, Hq2, sh2)
    torch.cuda.synchronize()
    n = int(offs[E])
    q1, q2 = Hq1.cpu().numpy()[:n], Hq2.cpu().numpy()[:n]
    s1, s2 = sh1.cpu().numpy()[:n], sh2.cpu().numpy()[:n]
    assert np.array_equal(q1, q2), f"{int((q1 != q2).sum())} codes differ from the unfused chain"
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    # the epilogue's SiLU-requant against the oracle's, on the chain's gate/up values
    nflip = 0
    qg = q2.astype(np.int64)
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        qr, sr = O.quant_act_static(h[a:b].astype(np.float32), s_e[e])
        assert np.array_equal(s2[a:b].view(np.uint32), sr.view(np.uint32))
        diff = np.abs(qg[a:b] - qr.astype(np.int64))
        assert diff.max() <= 1
        if diff.max() == 0:
            continue
        t = h[a:b] / np.float64(s_e[e])
        near = (np.abs(np.abs(t - np.floor(t)) - 0.5) < SILU_TIE_WINDOW) & (np.abs(t) < 127.5)
        assert np.all(near[diff > 0])
        nflip += int((diff > 0).sum())
    sat = int((np.abs(qg) == 127).sum())
    _print(f"  rows {n} I {I}: bit-exact with the chain; {nflip} near-tie flips against the oracle; "
           f"{sat} saturated codes")


@pytest.mark.parametrize("T,E,k,K,I,g,asym,gather,route", [
    (40, 8, 2, 1024, 256, 128, False, True, "streaming, 16-row tiles, gathered rows"),
    (40, 8, 2, 1024, 256, 64, True, False, "streaming, 16-row tiles, sorted rows"),
    (300, 4, 2, 512, 80, 64, True, True, "128-row tiles and streaming, 32-row tiles; I % 64 != 0"),
    (600, 4, 2, 1024, 144, 64, False, True, "128-row tiles, g = 64, symmetric, gathered rows"),
    (600, 4, 2, 512, 80, 64, True, False, "128-row tiles, g = 64, sorted rows"),
    (600, 4, 2, 512, 208, 128, False, True, "128-row tiles, g = 128, gathered rows"),
    (20, 16, 4, 6144, 128, 128, True, False, "K-slice, 16-row tiles"),
    (64, 4, 2, 6144, 96, 64, False, True, "chunked decode kernel, 32-row tiles"),
    (20, 16, 4, 9216, 64, 128, False, False, "chunked decode kernel, 16-row tiles, K > 8192"),
    (3, 5, 1, 256, 16, 64, False, True, "one h tile; empty experts"),
])
def test_moe_gemm_silu_static_matches_chain(T, E, k, K, I, g, asym, gather, route):
    _print(f"fused gate/up + static SiLU-requant: T={T} E={E} k={k} K={K} I={I} g={g} asym={asym} ({route})")
    _fused_vs_chain(T, E, k, K, I, g, asym, seed=T + K + I, gather=gather)


def test_moe_gemm_silu_static_degenerate_scales():
    """An expert whose scale is 0 and one whose scale is +Inf: zero codes, the scale passed through."""
    _print("fused gate/up + static SiLU-requant: degenerate expert scales")
    _fused_vs_chain(40, 8, 2, 512, 64, 128, False, 77, gather=True, bad_scales=True)


@pytest.mark.parametrize("name", ["c4", "c5_8tok"])
def test_moe_gemm_silu_static_full_shapes(name):
    """The 64-expert top-6 gate/up at full size (Zipf routing: experts with many rows run on
    128-row MFMA tiles) and the 256-expert gate/up (K = 7168, I = 2048) on 8 tokens."""
    if name == "c4":
        c = W.C4
        _print(f"fused gate/up + static SiLU-requant: {c.name} full")
        _fused_vs_chain(c.T, c.E, c.topk, c.H, c.I, c.group_size, c.asymmetric, 4, gather=False, zipf=c.zipf_s)
    else:
        c = W.C5
        _print(f"fused gate/up + static SiLU-requant: {c.name} on 8 tokens")
        _fused_vs_chain(8, c.E, c.topk, c.H, c.I, c.group_size, c.asymmetric, 5, gather=True)
