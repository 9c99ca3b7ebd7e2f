"""MI355X-native W4A8 linear / MoE-expert library: thin Python binding of libw4a8.so.

Every function here only marshals arguments to the C ABI declared in include/w4a8.h (same
names); all arithmetic runs in the library (host pack) or its gfx950 kernels.  PyTorch is
used for device memory and streams only.  There is no CPU fallback: if the library is not
built, or the GPU path is asked for without a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a8.so")

W4A8_OK, W4A8_EINVAL, W4A8_ESIZE, W4A8_EUNSUPPORTED, W4A8_EHIP = 0, -1, -2, -3, -4
W4A8_OUT_BF16, W4A8_OUT_F32 = 0, 1
HEADER_BYTES = 256

EXPORTED = [
    "w4a8_packed_size", "w4a8_pack", "w4a8_pack_codes", "w4a8_unpack_codes", "w4a8_blob_check",
    "w4a8_quant_act", "w4a8_quant_act_smooth", "w4a8_gemm", "w4a8_linear", "w4a8_gemm_partials", "w4a8_moe_align",
    "w4a8_moe_gemm",
    "w4a8_moe_gemm_silu_static",
    "w4a8_silu_mul_quant", "w4a8_moe_combine", "w4a8_moe_workspace_size", "w4a8_moe_forward",
    "w4a8_quant_act_static", "w4a8_moe_quant_static", "w4a8_silu_mul_quant_static",
    "w4a8_moe_static_workspace_size", "w4a8_moe_forward_static", "w4a8_moe_forward_sets", "w4a8_moe_forward_noalloc",
    "w4a16_gemm", "w4a16_kernel_name",
    "w4a8_kernel_name", "w4a8_status_string", "w4a8_version",
]


class W4A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class WDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("asymmetric", ctypes.c_int32), ("weight_bits", ctypes.c_int32), ("scale_bits", ctypes.c_int32)]

    def __repr__(self):
        return (f"WDesc(K={self.K}, N={self.N}, group_size={self.group_size}, asymmetric={self.asymmetric}, "
                f"weight_bits={self.weight_bits}, scale_bits={self.scale_bits})")


class ExpertSet(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("gu_blobs", ctypes.c_void_p), ("gu_stride", ctypes.c_size_t),
                ("gu_desc", ctypes.POINTER(WDesc)), ("d_blobs", ctypes.c_void_p), ("d_stride", ctypes.c_size_t),
                ("d_desc", ctypes.POINTER(WDesc))]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4a8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m moe_token_int8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, SZ, VP = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
        DP = ctypes.POINTER(WDesc)
        sig = {
            "w4a8_packed_size": (SZ, [DP]),
            "w4a8_pack": (I, [DP, P, P, SZ]),
            "w4a8_pack_codes": (I, [DP, P, P, P, P, SZ]),
            "w4a8_unpack_codes": (I, [P, SZ, DP, P, P, P]),
            "w4a8_blob_check": (I, [P, SZ, DP]),
            "w4a8_quant_act": (I, [P, I, I, I, P, P, VP]),
            "w4a8_quant_act_smooth": (I, [P, I, I, I, P, P, P, VP]),
            "w4a8_gemm": (I, [P, P, I, P, DP, P, I, I, VP]),
            "w4a8_linear": (I, [P, I, I, I, P, DP, P, I, I, P, P, VP]),
            "w4a8_gemm_partials": (I, [P, I, P, DP, P, VP]),
            "w4a8_moe_align": (I, [P, I, I, I, P, P, P, VP]),
            "w4a8_moe_gemm": (I, [P, P, P, I, P, I, I, I, P, SZ, DP, P, I, VP]),
            "w4a8_moe_gemm_silu_static": (I, [P, P, P, I, P, I, I, I, P, SZ, DP, P, P, P, VP]),
            "w4a8_silu_mul_quant": (I, [P, I, I, P, P, VP]),
            "w4a8_moe_combine": (I, [P, P, P, I, I, I, P, VP]),
            "w4a8_moe_workspace_size": (SZ, [I, I, I, I, I]),
            "w4a8_moe_forward": (I, [P, P, P, I, I, I, P, SZ, DP, P, SZ, DP, P, SZ, P, VP]),
            "w4a8_quant_act_static": (I, [P, I, I, I, P, P, P, VP]),
            "w4a8_moe_quant_static": (I, [P, I, I, I, P, I, P, I, P, P, P, VP]),
            "w4a8_silu_mul_quant_static": (I, [P, I, I, P, I, P, P, P, VP]),
            "w4a8_moe_static_workspace_size": (SZ, [I, I, I, I, I]),
            "w4a8_moe_forward_static": (I, [P, P, P, I, I, I, P, SZ, DP, P, SZ, DP, P, P, P, SZ, P, VP]),
            "w4a8_moe_forward_sets": (I, [P, P, P, I, I, ctypes.POINTER(ExpertSet), I, P, SZ, P, VP]),
            "w4a8_moe_forward_noalloc": (I, [P, P, P, I, I, I, P, SZ, DP, P, SZ, DP, P, VP]),
            "w4a8_kernel_name": (ctypes.c_char_p, [DP, I]),
            "w4a16_gemm": (I, [P, I, I, P, DP, P, I, I, VP]),
            "w4a16_kernel_name": (ctypes.c_char_p, [DP, I]),
            "w4a8_status_string": (ctypes.c_char_p, [I]),
            "w4a8_version": (I, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().w4a8_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != W4A8_OK:
        raise W4A8Error(status, where)


def desc(K: int, N: int, group_size: int, asymmetric: bool, bits: int = 4, scale_bits: int = 32) -> WDesc:
    """Weight descriptor; bits = 8 selects the symmetric INT8-weight (W8A8) form, scale_bits = 16
    binary16 group scales."""
    return WDesc(int(K), int(N), int(group_size), int(bool(asymmetric)), int(bits), int(scale_bits))


def _ptr(x) -> int | None:
    """Data pointer of a torch tensor or numpy array (None passes NULL)."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not (hasattr(t, "is_cuda") and t.is_cuda):
            raise ValueError("GPU entry points take device tensors")


# ------------------------------------------------------------------------------ host side
def w4a8_packed_size(d: WDesc) -> int:
    return int(lib().w4a8_packed_size(ctypes.byref(d)))


def w4a8_pack(d: WDesc, W: np.ndarray) -> np.ndarray:
    """RTN-quantize and pack float32 W[K, N] on the host; returns the blob (uint8)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.shape != (d.K, d.N):
        raise ValueError(f"W shape {W.shape} does not match {d}")
    n = w4a8_packed_size(d)
    if n == 0:
        raise W4A8Error(W4A8_EINVAL, "w4a8_packed_size")
    blob = np.empty(n, dtype=np.uint8)
    _check(lib().w4a8_pack(ctypes.byref(d), _ptr(W), _ptr(blob), n), "w4a8_pack")
    return blob


def w4a8_pack_codes(d: WDesc, codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray | None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    if zeros is not None:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    n = w4a8_packed_size(d)
    if n == 0:
        raise W4A8Error(W4A8_EINVAL, "w4a8_packed_size")
    blob = np.empty(n, dtype=np.uint8)
    _check(lib().w4a8_pack_codes(ctypes.byref(d), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(blob), n),
           "w4a8_pack_codes")
    return blob


def w4a8_unpack_codes(blob: np.ndarray):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    d = WDesc()
    st = lib().w4a8_unpack_codes(_ptr(blob), blob.nbytes, ctypes.byref(d), None, None, None)
    _check(st, "w4a8_unpack_codes")
    G = d.K // d.group_size
    codes = np.empty((d.K, d.N), np.int8)
    scales = np.empty((G, d.N), np.float32)
    zeros = np.empty((G, d.N), np.uint8) if d.asymmetric else None
    _check(lib().w4a8_unpack_codes(_ptr(blob), blob.nbytes, ctypes.byref(d), _ptr(codes), _ptr(scales),
                                   _ptr(zeros)), "w4a8_unpack_codes")
    return d, codes, scales, zeros


def w4a8_blob_check(blob: np.ndarray, d: WDesc) -> None:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    _check(lib().w4a8_blob_check(_ptr(blob), blob.nbytes, ctypes.byref(d)), "w4a8_blob_check")


def w4a8_kernel_name(d: WDesc, M: int) -> str:
    return lib().w4a8_kernel_name(ctypes.byref(d), int(M)).decode()


def w4a8_moe_workspace_size(T: int, k: int, H: int, I: int, E: int) -> int:
    return int(lib().w4a8_moe_workspace_size(T, k, H, I, E))


def w4a8_moe_static_workspace_size(T: int, k: int, H: int, I: int, E: int) -> int:
    return int(lib().w4a8_moe_static_workspace_size(T, k, H, I, E))


def w4a8_version() -> int:
    return int(lib().w4a8_version())


# ------------------------------------------------------------------------------ GPU side
def w4a8_quant_act(X, Xq, sx, stream=None) -> None:
    """X: bf16 [M, K] (row stride X.stride(0)); Xq: int8 [M, K]; sx: float32 [M]."""
    _require_cuda(X, Xq, sx)
    M, K = X.shape
    _check(lib().w4a8_quant_act(_ptr(X), M, K, X.stride(0), _ptr(Xq), _ptr(sx), _stream(stream)),
           "w4a8_quant_act")


def w4a8_quant_act_smooth(X, inv_alpha, Xq, sx, stream=None) -> None:
    """w4a8_quant_act of X diag(alpha)^-1; inv_alpha: float32 [K] on the device."""
    _require_cuda(X, inv_alpha, Xq, sx)
    M, K = X.shape
    _check(lib().w4a8_quant_act_smooth(_ptr(X), M, K, X.stride(0), _ptr(inv_alpha), _ptr(Xq), _ptr(sx),
                                       _stream(stream)), "w4a8_quant_act_smooth")


def w4a8_quant_act_static(X, s, Xq, sx, stream=None) -> None:
    """Quantize every row of X (bf16 [M, K]) with the one calibrated scale s (float32 [1] on
    the device); sx[m] receives s."""
    _require_cuda(X, s, Xq, sx)
    M, K = X.shape
    _check(lib().w4a8_quant_act_static(_ptr(X), M, K, X.stride(0), _ptr(s), _ptr(Xq), _ptr(sx), _stream(stream)),
           "w4a8_quant_act_static")


def w4a8_moe_quant_static(X, k: int, sorted_rows, expert_offsets, E: int, s, Xq, sx, stream=None) -> None:
    """Routed rows in expert-sorted order: row r quantizes token sorted_rows[r] // k of X with the
    scale s[e] of its expert; Xq int8 [T*k, H], sx float32 [T*k]."""
    _require_cuda(X, sorted_rows, expert_offsets, s, Xq, sx)
    T, H = X.shape
    _check(lib().w4a8_moe_quant_static(_ptr(X), T, H, X.stride(0), _ptr(sorted_rows), int(k), _ptr(expert_offsets),
                                       int(E), _ptr(s), _ptr(Xq), _ptr(sx), _stream(stream)), "w4a8_moe_quant_static")


def w4a8_gemm(Xq, sx, blob_dev, d: WDesc, Y, out_dtype: int = W4A8_OUT_BF16, stream=None) -> None:
    _require_cuda(Xq, sx, blob_dev, Y)
    _check(lib().w4a8_gemm(_ptr(Xq), _ptr(sx), Xq.shape[0], _ptr(blob_dev), ctypes.byref(d), _ptr(Y),
                           Y.stride(0), int(out_dtype), _stream(stream)), "w4a8_gemm")


def w4a8_linear(X, blob_dev, d: WDesc, Y, Xq, sx, out_dtype: int = W4A8_OUT_BF16, stream=None) -> None:
    """Quantize X (bf16 [M, K]) per token and multiply: Y = GEMM(quant(X)); Xq/sx receive the
    activation codes and scales."""
    _require_cuda(X, blob_dev, Y, Xq, sx)
    M, K = X.shape
    _check(lib().w4a8_linear(_ptr(X), M, K, X.stride(0), _ptr(blob_dev), ctypes.byref(d), _ptr(Y), Y.stride(0),
                             int(out_dtype), _ptr(Xq), _ptr(sx), _stream(stream)), "w4a8_linear")


def w4a16_gemm(X, blob_dev, d: WDesc, Y, out_dtype: int = W4A8_OUT_BF16, stream=None) -> None:
    """W4A16 sibling: Y = X W with bfloat16 activations and the blob's 4-bit weights dequantized in
    the kernel (no activation quantization)."""
    _require_cuda(X, blob_dev, Y)
    M = X.shape[0]
    _check(lib().w4a16_gemm(_ptr(X), int(M), int(X.stride(0)), _ptr(blob_dev), ctypes.byref(d), _ptr(Y),
                            int(Y.stride(0)), int(out_dtype), _stream(stream)), "w4a16_gemm")


def w4a16_kernel_name(d: WDesc, M: int) -> str:
    return lib().w4a16_kernel_name(ctypes.byref(d), int(M)).decode()


def w4a8_gemm_partials(Xq, blob_dev, d: WDesc, P, stream=None) -> None:
    _require_cuda(Xq, blob_dev, P)
    _check(lib().w4a8_gemm_partials(_ptr(Xq), Xq.shape[0], _ptr(blob_dev), ctypes.byref(d), _ptr(P),
                                    _stream(stream)), "w4a8_gemm_partials")


def w4a8_moe_align(topk_ids, E: int, sorted_rows, expert_offsets, inv, stream=None) -> None:
    _require_cuda(topk_ids, sorted_rows, expert_offsets, inv)
    T, k = topk_ids.shape
    _check(lib().w4a8_moe_align(_ptr(topk_ids), T, k, int(E), _ptr(sorted_rows), _ptr(expert_offsets),
                                _ptr(inv), _stream(stream)), "w4a8_moe_align")


def w4a8_moe_gemm(Xq, sx, gather, k: int, expert_offsets, E: int, rows: int, blobs_dev, expert_stride: int,
                  d: WDesc, Y, out_dtype: int = W4A8_OUT_BF16, stream=None) -> None:
    _require_cuda(Xq, sx, gather, expert_offsets, blobs_dev, Y)
    src_rows = int(Xq.shape[0])
    if sx.numel() < src_rows:
        raise ValueError("sx must hold one scale per row of Xq")
    _check(lib().w4a8_moe_gemm(_ptr(Xq), _ptr(sx), _ptr(gather), int(k), _ptr(expert_offsets), int(E), int(rows),
                               src_rows, _ptr(blobs_dev), int(expert_stride), ctypes.byref(d), _ptr(Y),
                               int(out_dtype), _stream(stream)), "w4a8_moe_gemm")


def w4a8_moe_gemm_silu_static(Xq, sx, gather, k: int, expert_offsets, E: int, rows: int, blobs_dev,
                              expert_stride: int, d: WDesc, s, Hq, sh, stream=None) -> None:
    """Grouped gate/up GEMM with the static SiLU-requant in its epilogue: Hq [rows, N/2], sh [rows]."""
    _require_cuda(Xq, sx, gather, expert_offsets, blobs_dev, s, Hq, sh)
    src_rows = int(Xq.shape[0])
    if sx.numel() < src_rows:
        raise ValueError("sx must hold one scale per row of Xq")
    _check(lib().w4a8_moe_gemm_silu_static(_ptr(Xq), _ptr(sx), _ptr(gather), int(k), _ptr(expert_offsets), int(E),
                                           int(rows), src_rows, _ptr(blobs_dev), int(expert_stride), ctypes.byref(d),
                                           _ptr(s), _ptr(Hq), _ptr(sh), _stream(stream)),
           "w4a8_moe_gemm_silu_static")


def w4a8_silu_mul_quant(GU, Hq, sh, stream=None) -> None:
    _require_cuda(GU, Hq, sh)
    R, I2 = GU.shape
    _check(lib().w4a8_silu_mul_quant(_ptr(GU), R, I2 // 2, _ptr(Hq), _ptr(sh), _stream(stream)),
           "w4a8_silu_mul_quant")


def w4a8_silu_mul_quant_static(GU, expert_offsets, E: int, s, Hq, sh, stream=None) -> None:
    _require_cuda(GU, expert_offsets, s, Hq, sh)
    R, I2 = GU.shape
    _check(lib().w4a8_silu_mul_quant_static(_ptr(GU), R, I2 // 2, _ptr(expert_offsets), int(E), _ptr(s), _ptr(Hq),
                                            _ptr(sh), _stream(stream)), "w4a8_silu_mul_quant_static")


def w4a8_moe_combine(Yd, inv, topk_w, out, stream=None) -> None:
    _require_cuda(Yd, inv, topk_w, out)
    T, k = inv.shape
    H = Yd.shape[1]
    _check(lib().w4a8_moe_combine(_ptr(Yd), _ptr(inv), _ptr(topk_w), T, k, H, _ptr(out), _stream(stream)),
           "w4a8_moe_combine")


def w4a8_moe_forward(X, topk_ids, topk_w, E: int, gu_blobs, gu_stride: int, gu_desc: WDesc, d_blobs,
                     d_stride: int, d_desc: WDesc, workspace, out, stream=None) -> None:
    _require_cuda(X, topk_ids, topk_w, gu_blobs, d_blobs, workspace, out)
    T, k = topk_ids.shape
    _check(lib().w4a8_moe_forward(_ptr(X), _ptr(topk_ids), _ptr(topk_w), T, k, int(E), _ptr(gu_blobs),
                                  int(gu_stride), ctypes.byref(gu_desc), _ptr(d_blobs), int(d_stride),
                                  ctypes.byref(d_desc), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _ptr(out), _stream(stream)), "w4a8_moe_forward")


def w4a8_moe_forward_noalloc(X, topk_ids, topk_w, E: int, gu_blobs, gu_stride: int, gu_desc: WDesc, d_blobs,
                             d_stride: int, d_desc: WDesc, out, stream=None) -> None:
    """w4a8_moe_forward on the library's own device scratch (no workspace argument; the call
    allocates nothing).  Calls that overlap on one GPU race: serialize them."""
    _require_cuda(X, topk_ids, topk_w, gu_blobs, d_blobs, out)
    T, k = topk_ids.shape
    _check(lib().w4a8_moe_forward_noalloc(_ptr(X), _ptr(topk_ids), _ptr(topk_w), T, k, int(E), _ptr(gu_blobs),
                                          int(gu_stride), ctypes.byref(gu_desc), _ptr(d_blobs), int(d_stride),
                                          ctypes.byref(d_desc), _ptr(out), _stream(stream)),
           "w4a8_moe_forward_noalloc")


def w4a8_moe_forward_static(X, topk_ids, topk_w, E: int, gu_blobs, gu_stride: int, gu_desc: WDesc, d_blobs,
                            d_stride: int, d_desc: WDesc, s_gu, s_dn, workspace, out, stream=None) -> None:
    """w4a8_moe_forward with static per-expert activation scales s_gu, s_dn (float32 [E] on the
    device); workspace of w4a8_moe_static_workspace_size bytes."""
    _require_cuda(X, topk_ids, topk_w, gu_blobs, d_blobs, s_gu, s_dn, workspace, out)
    T, k = topk_ids.shape
    _check(lib().w4a8_moe_forward_static(_ptr(X), _ptr(topk_ids), _ptr(topk_w), T, k, int(E), _ptr(gu_blobs),
                                         int(gu_stride), ctypes.byref(gu_desc), _ptr(d_blobs), int(d_stride),
                                         ctypes.byref(d_desc), _ptr(s_gu), _ptr(s_dn), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)),
           "w4a8_moe_forward_static")


def w4a8_moe_forward_sets(X, topk_ids, topk_w, sets, workspace, out, stream=None) -> None:
    """One MoE layer whose experts come in format classes: `sets` is a list of
    (DeviceWeights gate/up, DeviceWeights down) pairs, experts numbered set by set."""
    _require_cuda(X, topk_ids, topk_w, workspace, out)
    T, k = topk_ids.shape
    arr = (ExpertSet * len(sets))()
    keep = []
    for i, (gu, dn) in enumerate(sets):
        if gu.experts != dn.experts:
            raise ValueError("gate/up and down sets must hold the same experts")
        gd, dd = WDesc(*[getattr(gu.desc, f) for f, _ in WDesc._fields_]), \
            WDesc(*[getattr(dn.desc, f) for f, _ in WDesc._fields_])
        keep += [gd, dd]
        arr[i] = ExpertSet(gu.experts, _ptr(gu.blob), gu.stride, ctypes.pointer(gd), _ptr(dn.blob), dn.stride,
                           ctypes.pointer(dd))
    _check(lib().w4a8_moe_forward_sets(_ptr(X), _ptr(topk_ids), _ptr(topk_w), T, k, arr, len(sets), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)),
           "w4a8_moe_forward_sets")


# ------------------------------------------------------------------------------ helpers
@dataclass
class DeviceWeights:
    """A packed blob (or E blobs back to back) resident on the device."""
    desc: WDesc
    blob: "object"          # torch uint8 cuda tensor
    stride: int             # bytes between experts (= packed size)
    experts: int = 1


def to_device(d: WDesc, blobs, device="cuda") -> DeviceWeights:
    """Copy one host blob or a list of host blobs (same desc) into one device buffer."""
    import torch
    if isinstance(blobs, np.ndarray):
        blobs = [blobs]
    n = w4a8_packed_size(d)
    for b in blobs:
        w4a8_blob_check(b, d)
    host = np.concatenate([np.ascontiguousarray(b[:n]) for b in blobs])
    dev = torch.from_numpy(host).to(device)
    return DeviceWeights(d, dev, n, len(blobs))


def experts_to_device(d: WDesc, E: int, blobs: dict, device="cuda") -> DeviceWeights:
    """E expert blobs of one desc in one zero-initialised device buffer; `blobs` maps expert
    id -> host blob and may omit experts that receive no rows (their bytes stay zero and
    are never read)."""
    import torch
    n = w4a8_packed_size(d)
    dev = torch.zeros(E * n, dtype=torch.uint8, device=device)
    for e, b in blobs.items():
        w4a8_blob_check(b, d)
        dev[e * n:(e + 1) * n].copy_(torch.from_numpy(np.ascontiguousarray(b[:n])))
    return DeviceWeights(d, dev, n, E)
