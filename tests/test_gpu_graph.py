"""MoE layers captured into a HIP graph.  The format classes of w4a8_moe_forward_sets run in one
launch pair per GEMM (up to four sets, K <= 4096) or else side by side on helper streams, forked
from the caller's stream and joined back with events; a graph captured on the caller's stream
must hold those branches.  Each test replays the graph several
times, with eager work and synchronizations in between, and every replay must reproduce the
eager output bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import workloads as W
from gpu_cases import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _layer(T, E, k, H, I, seed):
    cfg = W.MoEConfig("graph", T, H, I, E, k, 128, False, seed, zipf_s=1.1)
    ids, w = W.moe_routing(cfg)
    X = W.moe_activations(cfg).to(DEV)
    return cfg, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), X


def _experts(seed, E, K, N, g, asym):
    d = L.desc(K, N, g, asym)
    host = {e: L.w4a8_pack_codes(d, *W.random_codes(seed * 31 + e, K, N, g, asym)) for e in range(E)}
    return d, L.experts_to_device(d, E, host)


def _replays_match(fn, out, n=4):
    fn()                                             # eager (also creates the helper streams)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager output"
        fn()                                         # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_moe_forward_graph_with_hot_experts():
    """300 tokens over 4 experts, top-2: every expert has >= 128 rows (the 128-row MFMA tiles)."""
    _print("graph: moe_forward, experts with many rows")
    cfg, ids, w, X = _layer(300, 4, 2, 512, 256, 11)
    gud, gdev = _experts(3, cfg.E, cfg.H, 2 * cfg.I, 128, False)
    ddv, ddev = _experts(4, cfg.E, cfg.I, cfg.H, 128, False)
    ws = torch.empty(L.w4a8_moe_workspace_size(cfg.T, cfg.topk, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    _replays_match(lambda: L.w4a8_moe_forward(X, ids, w, cfg.E, gdev.blob, gdev.stride, gud, ddev.blob, ddev.stride,
                                              ddv, ws, out), out)


def test_moe_forward_sets_graph_two_classes():
    """Two format classes in one launch pair per GEMM, each with experts of many rows."""
    _print("graph: moe_forward_sets, two classes")
    cfg, ids, w, X = _layer(400, 6, 2, 512, 256, 12)
    sets = []
    for i, g in enumerate((128, 64)):
        gd, gdev = _experts(20 + i, 3, cfg.H, 2 * cfg.I, g, i == 1)
        dd, ddev = _experts(30 + i, 3, cfg.I, cfg.H, g, i == 1)
        sets.append((gdev, ddev))
    ws = torch.empty(L.w4a8_moe_workspace_size(cfg.T, cfg.topk, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    _replays_match(lambda: L.w4a8_moe_forward_sets(X, ids, w, sets, ws, out), out)


def test_moe_forward_sets_graph_five_classes():
    """Five format classes: one launch per set, sets 1-4 on the helper streams."""
    _print("graph: moe_forward_sets, five classes")
    cfg, ids, w, X = _layer(400, 10, 2, 512, 256, 13)
    sets = []
    for i, (n, g, asym) in enumerate(((2, 128, False), (2, 64, True), (2, 128, True), (2, 64, False), (2, 128, False))):
        gd, gdev = _experts(40 + i, n, cfg.H, 2 * cfg.I, g, asym)
        dd, ddev = _experts(50 + i, n, cfg.I, cfg.H, g, asym)
        sets.append((gdev, ddev))
    ws = torch.empty(L.w4a8_moe_workspace_size(cfg.T, cfg.topk, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    _replays_match(lambda: L.w4a8_moe_forward_sets(X, ids, w, sets, ws, out), out)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_decode_linear_graph(M):
    """The decode Linear (quantization + GEMM; at 32 rows the split-K-slice kernel, at 1 row the
    fused quantization) on the 4096 x 14336 projection, captured and replayed."""
    _print(f"graph: w4a8_linear M={M}")
    K, N = 4096, 14336
    d = L.desc(K, N, 128, False)
    host = L.w4a8_pack_codes(d, *W.random_codes(40 + M, K, N, 128, False))
    blob = torch.from_numpy(host).to(DEV)
    X = W.random_activations(50 + M, M, K, outlier_cols=4, outlier_scale=50.0).to(DEV)
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty(M, dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _replays_match(lambda: L.w4a8_linear(X, blob, d, out, Xq, sx), out)
