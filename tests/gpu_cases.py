"""Shared helpers of the GPU parity tests: input staging, oracle comparison gates."""
import numpy as np
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W

DEV = "cuda"


def bf16_ulp(x):
    """Spacing of the bfloat16 grid at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


# Near-tie window of the SiLU requantization, in units of the code t = h / s.
# The kernel computes h = RN(RN(g / RN(1 + expf(-g))) * u) in float32 from exact bfloat16 g, u.
# With expf within 1 ulp, the relative error of h against the exact value is at most
# 2^-23 (exp through 1 + e) + 3 * 2^-24 (three roundings) = 2.5 * 2^-23 ~ 3.0e-7.  At
# |t| <= 127 that moves t by <= 3.8e-5; the dynamic scale s = fl32(max|h| / 127) carries the same
# relative error (another 3.8e-5), and the oracle's own float32 rounding of h adds 127 * 2^-24 ~
# 7.6e-6.  Total < 8.4e-5, so a code may differ by one only where the float64 t lies within
# 1e-4 of a .5 boundary.
SILU_TIE_WINDOW = 1e-4


def gpu_quant(Xb: torch.Tensor):
    X = Xb.to(DEV)
    M, K = X.shape
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty((M,), dtype=torch.float32, device=DEV)
    L.w4a8_quant_act(X, Xq, sx)
    return Xq, sx


def check_float_output(y32, ybf, Y64, rel_tol=1e-3):
    """Gates for a GEMM output.
    1. float32 mode within rel_tol of the float64 oracle, relative to max(|Y64|, 1e-3 max|Y64|);
    2. the bfloat16 mode is the round-to-nearest-even of the float32 mode, bit for bit;
    3. bfloat16 mode vs the correctly rounded oracle: at most one bf16 step apart (plus the
       float32 error allowance), and normwise within rel_tol.
    Returns a dict of observed figures."""
    Y64 = np.asarray(Y64, np.float64)
    y32 = np.asarray(y32, np.float64)
    ybf = np.asarray(ybf, np.float32)
    finite = np.isfinite(Y64)
    assert np.array_equal(np.isfinite(y32), finite)
    scale = np.max(np.abs(Y64[finite])) if finite.any() else 1.0
    den = np.maximum(np.abs(Y64), 1e-3 * scale)
    rel = np.max(np.abs(y32 - Y64)[finite] / den[finite]) if finite.any() else 0.0
    assert rel <= rel_tol, rel
    rne = O.bf16_rne(y32)
    same = (rne.view(np.uint32) == ybf.view(np.uint32)) | (np.isnan(rne) & np.isnan(ybf))
    assert same.all(), int((~same).sum())
    ref = O.bf16_rne(Y64)
    diff = np.abs(ybf.astype(np.float64) - ref)[finite]
    allow = bf16_ulp(ref[finite]) + 1e-5 * scale
    assert np.all(diff <= allow), float(np.max(diff - allow))
    nw = np.linalg.norm(diff) / max(np.linalg.norm(Y64[finite]), 1e-30)
    assert nw <= rel_tol, nw
    mism = int(np.count_nonzero(diff))
    return dict(max_rel_f32=float(rel), normwise_bf16=float(nw), bf16_mismatch=mism, n=int(finite.sum()))


def device_blob(d, host_blob):
    return torch.from_numpy(np.ascontiguousarray(host_blob)).to(DEV)


def random_expert_set(seed, E, K, N, g, asym):
    """Per-expert random well-formed codes (no float weights), generated on demand."""
    def make(e):
        return W.random_codes(seed * 1009 + e, K, N, g, asym)
    return make


# ---------------------------------------------------------------- MoE layer helpers
def moe_experts_rtn(cfg, experts_touched):
    """Float weights quantized by the oracle (for the oracle) and packed by the library."""
    dgu = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric)
    dd = L.desc(cfg.I, cfg.H, cfg.group_size, cfg.asymmetric)
    host_gu, host_d, qw = {}, {}, {}
    for e in sorted(experts_touched):
        Wgu, Wd = W.expert_weights(cfg, e)
        host_gu[e] = L.w4a8_pack(dgu, Wgu)
        host_d[e] = L.w4a8_pack(dd, Wd)
        qw[e] = O.quant_weight(Wgu, cfg.group_size, cfg.asymmetric) + \
            O.quant_weight(Wd, cfg.group_size, cfg.asymmetric)
    return (dgu, dd, L.experts_to_device(dgu, cfg.E, host_gu), L.experts_to_device(dd, cfg.E, host_d), qw)


def moe_experts_codes(cfg, experts_touched, seed):
    """Random well-formed codes per expert (sizes whose float weights are too slow to draw)."""
    dgu = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric)
    dd = L.desc(cfg.I, cfg.H, cfg.group_size, cfg.asymmetric)
    host_gu, host_d, qw = {}, {}, {}
    for e in sorted(experts_touched):
        cg = W.random_codes(seed * 1009 + e, cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric)
        cd = W.random_codes(seed * 2003 + e, cfg.I, cfg.H, cfg.group_size, cfg.asymmetric)
        host_gu[e] = L.w4a8_pack_codes(dgu, *cg)
        host_d[e] = L.w4a8_pack_codes(dd, *cd)
        qw[e] = cg + cd
    return (dgu, dd, L.experts_to_device(dgu, cfg.E, host_gu), L.experts_to_device(dd, cfg.E, host_d), qw)


def run_moe_forward(cfg, Xb, ids, w, gud, dd_):
    T, k = ids.shape
    ws = torch.empty(L.w4a8_moe_workspace_size(T, k, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_forward(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E,
                       gud.blob, gud.stride, gud.desc, dd_.blob, dd_.stride, dd_.desc, ws, out)
    return out, ws


def check_moe(out, ref, qw, group_size, flips_per_row=2):
    """End-to-end gate against the oracle's own bf16 output.

    The stages are pinned one by one above; end to end, two things may legitimately differ:
    bf16 roundings of intermediate outputs (one step when a value sits on a rounding
    boundary), and the requantization of silu(gate)*up, where a near-tie code can move by
    +-1 (the GPU's expf and the oracle's float64 exp differ by ulps).  One such flip in
    routed row r moves out[t, n] by at most w[t, j] * sh[r] * max_k |s_d (q - z)|[k, n].
    Bound per element: 2 bf16 steps + flips_per_row of those for each routed row; normwise
    1e-3 against the float64 output."""
    got = out.float().cpu().numpy().astype(np.float64)
    ref_bf = ref["out"].astype(np.float64)
    o64 = ref["out64"]
    inv, sh = ref["inv"], ref["sh"].astype(np.float64)
    T, k = inv.shape
    srt, offs = ref["sorted_rows"], ref["offsets"]
    flip = np.zeros_like(o64)
    colmax = {}
    for e, wts in qw.items():
        cd, sd, zd = wts[3:]
        deq = O.dequant_weight(cd, sd, zd, group_size if np.ndim(group_size) == 0 else group_size[e])
        colmax[e] = np.max(np.abs(deq), axis=0)
    ids = np.empty(T * k, np.int64)
    for e in range(len(offs) - 1):
        ids[srt[offs[e]:offs[e + 1]]] = e
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            e = ids[t * k + j]
            flip[t] += abs(ref["topk_w"][t, j]) * sh[r] * colmax[e]
    rms = np.sqrt(np.mean(o64 ** 2))
    nw = np.linalg.norm(got - ref_bf) / np.linalg.norm(o64)
    err = np.abs(got - ref_bf)
    allow = 2 * bf16_ulp(ref_bf) + flips_per_row * flip
    stats = dict(normwise=float(nw), frac_bitexact=float(np.mean(got == ref_bf)),
                 frac_within_1ulp=float(np.mean(err <= bf16_ulp(ref_bf))),
                 max_err_over_rms=float(np.max(err) / rms), max_err_over_allow=float(np.max(err / allow)))
    print(stats, flush=True)
    assert nw < 1e-3, stats
    assert np.all(err <= allow), stats
    return stats


def sample_tokens(T, n, seed):
    """n distinct token indices of a T-token batch, always including the first and the last
    (sorted).  The MoE layer is independent per token once the routing is fixed, so the
    oracle runs on these tokens only while the GPU runs the whole batch."""
    rs = np.random.default_rng(seed)
    mid = rs.choice(np.arange(1, T - 1), size=max(0, n - 2), replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid])).astype(np.int64)
