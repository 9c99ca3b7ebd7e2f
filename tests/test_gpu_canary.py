"""Guard regions around every output of the GPU entry points, and run-twice determinism.

Each output (and the MoE workspace) is a view into a larger buffer whose guard bytes before and
after hold a fixed pattern; after the call the guards must be unchanged, so no kernel writes
outside the rows and columns it owns (ragged tiles included).  Every entry point is then called
twice on the same inputs and must give bit-identical outputs (the kernels fix every summation
order; the format classes of w4a8_moe_forward_sets, in one launch or on helper streams, must
not change that)."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import workloads as W
from gpu_cases import DEV, device_blob

pytestmark = pytest.mark.gpu

GUARD = 4096            # bytes on each side (a multiple of 256, so views keep their alignment)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


class Guarded:
    """A tensor of `shape`/`dtype` inside a byte buffer with guard regions on both sides."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n
        self.buf = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(*shape)

    def intact(self):
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes:]
        return bool((head == PATTERN).all()) and bool((tail == PATTERN).all())


def _weights(K, N, g, asym, seed):
    d = L.desc(K, N, g, asym)
    return d, device_blob(d, L.w4a8_pack_codes(d, *W.random_codes(seed, K, N, g, asym)))


@pytest.mark.parametrize("M,K,N,g,asym", [(5, 1024, 80, 128, False), (23, 512, 200, 64, True),
                                          (300, 512, 200, 128, True), (1, 4096, 48, 128, False),
                                          # the split decode kernel: 16- and 32-row tiles, ragged N and K
                                          (9, 3072, 200, 64, True), (29, 4096, 72, 128, False),
                                          (20, 2176, 40, 64, False)])
def test_gemm_outputs_guarded_and_deterministic(M, K, N, g, asym):
    _print(f"guards: quant + gemm + linear + w4a16 M={M} K={K} N={N} g={g} asym={asym}")
    d, blob = _weights(K, N, g, asym, M + K + N)
    X = W.random_activations(M, M, K, outlier_cols=2, outlier_scale=20.0).to(DEV)
    Xq, sx = Guarded((M, K), torch.int8), Guarded((M,), torch.float32)
    L.w4a8_quant_act(X, Xq.t, sx.t)
    outs = {}
    for name, dt, od in (("bf16", torch.bfloat16, L.W4A8_OUT_BF16), ("f32", torch.float32, L.W4A8_OUT_F32)):
        ys = []
        for _ in range(2):
            Y = Guarded((M, N), dt)
            L.w4a8_gemm(Xq.t, sx.t, blob, d, Y.t, od)
            torch.cuda.synchronize()
            assert Y.intact(), f"w4a8_gemm ({name}) wrote outside its output"
            ys.append(Y.t.clone())
        assert torch.equal(ys[0], ys[1]), f"w4a8_gemm ({name}) differs between two runs"
        outs[name] = ys[0]
    assert Xq.intact() and sx.intact()
    # the fused entry point (quantization + GEMM) and the W4A16 sibling
    ys = []
    for _ in range(2):
        Y, Xq2, sx2 = Guarded((M, N), torch.bfloat16), Guarded((M, K), torch.int8), Guarded((M,), torch.float32)
        L.w4a8_linear(X, blob, d, Y.t, Xq2.t, sx2.t)
        torch.cuda.synchronize()
        assert Y.intact() and Xq2.intact() and sx2.intact(), "w4a8_linear wrote outside its outputs"
        ys.append(Y.t.clone())
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], outs["bf16"])
    ys = []
    for _ in range(2):
        Y = Guarded((M, N), torch.bfloat16)
        L.w4a16_gemm(X, blob, d, Y.t)
        torch.cuda.synchronize()
        assert Y.intact(), "w4a16_gemm wrote outside its output"
        ys.append(Y.t.clone())
    assert torch.equal(ys[0], ys[1])


def _moe_case(T, E, k, H, I, g, asym, seed, zipf):
    cfg = W.MoEConfig("guard", T, H, I, E, k, g, asym, seed, zipf_s=zipf)
    ids, w = W.moe_routing(cfg)
    X = W.moe_activations(cfg).to(DEV)
    return cfg, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), X


def _experts(seed, E, K, N, g, asym):
    d = L.desc(K, N, g, asym)
    host = {e: L.w4a8_pack_codes(d, *W.random_codes(seed * 31 + e, K, N, g, asym)) for e in range(E)}
    return d, L.experts_to_device(d, E, host)


@pytest.mark.parametrize("T,E,k,H,I,g,asym,zipf", [(300, 6, 2, 512, 256, 128, False, 1.1),
                                                   (9, 16, 4, 256, 128, 64, True, 0.0)])
def test_moe_outputs_guarded_and_deterministic(T, E, k, H, I, g, asym, zipf):
    """The dynamic layer (experts with many rows on the 128-row MFMA tiles when T = 300), its workspace
    guarded too; the static layer with the fused SiLU-requant; two format classes side by side."""
    _print(f"guards: moe layers T={T} E={E} k={k} H={H} I={I} g={g} asym={asym}")
    cfg, ids, w, X = _moe_case(T, E, k, H, I, g, asym, 50 + T, zipf)
    gud, gdev = _experts(3, E, H, 2 * I, g, asym)
    ddv, ddev = _experts(4, E, I, H, g, asym)
    s_gu = torch.full((E,), 0.05, dtype=torch.float32, device=DEV)
    s_dn = torch.full((E,), 0.02, dtype=torch.float32, device=DEV)
    runs = {"dynamic": [], "static": [], "sets": []}
    for _ in range(2):
        ws = Guarded((L.w4a8_moe_workspace_size(T, k, H, I, E),), torch.uint8)
        out = Guarded((T, H), torch.bfloat16)
        L.w4a8_moe_forward(X, ids, w, E, gdev.blob, gdev.stride, gud, ddev.blob, ddev.stride, ddv, ws.t, out.t)
        torch.cuda.synchronize()
        assert out.intact() and ws.intact(), "w4a8_moe_forward wrote outside its output or workspace"
        runs["dynamic"].append(out.t.clone())
        ws = Guarded((L.w4a8_moe_static_workspace_size(T, k, H, I, E),), torch.uint8)
        out = Guarded((T, H), torch.bfloat16)
        L.w4a8_moe_forward_static(X, ids, w, E, gdev.blob, gdev.stride, gud, ddev.blob, ddev.stride, ddv, s_gu, s_dn,
                                  ws.t, out.t)
        torch.cuda.synchronize()
        assert out.intact() and ws.intact(), "w4a8_moe_forward_static wrote outside its output or workspace"
        runs["static"].append(out.t.clone())
        h = E // 2
        sets = [(L.DeviceWeights(gud, gdev.blob[:h * gdev.stride], gdev.stride, h),
                 L.DeviceWeights(ddv, ddev.blob[:h * ddev.stride], ddev.stride, h)),
                (L.DeviceWeights(gud, gdev.blob[h * gdev.stride:], gdev.stride, E - h),
                 L.DeviceWeights(ddv, ddev.blob[h * ddev.stride:], ddev.stride, E - h))]
        ws = Guarded((L.w4a8_moe_workspace_size(T, k, H, I, E),), torch.uint8)
        out = Guarded((T, H), torch.bfloat16)
        L.w4a8_moe_forward_sets(X, ids, w, sets, ws.t, out.t)
        torch.cuda.synchronize()
        assert out.intact() and ws.intact(), "w4a8_moe_forward_sets wrote outside its output or workspace"
        runs["sets"].append(out.t.clone())
    for name, (a, b) in runs.items():
        assert torch.equal(a, b), f"{name} layer differs between two runs"
    # the classes split the same experts: the same layer
    assert torch.equal(runs["sets"][0], runs["dynamic"][0])
