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
