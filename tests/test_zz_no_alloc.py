"""The MoE layer entry point that allocates nothing (its workspace is the library's own device
scratch), against w4a8_moe_forward with a caller workspace: bit-identical outputs on two calls in
a row, the second with fewer tokens and a different routing, so that the scratch holds the
first call's contents when the second one starts."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import workloads as W
from gpu_cases import DEV, moe_experts_rtn

pytestmark = pytest.mark.gpu


def _reference(cfg, Xb, ids, w, gud, ddv):
    T, k = ids.shape
    ws = torch.empty(L.w4a8_moe_workspace_size(T, k, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_forward(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E,
                       gud.blob, gud.stride, gud.desc, ddv.blob, ddv.stride, ddv.desc, ws, out)
    return out


def _noalloc(cfg, Xb, ids, w, gud, ddv):
    T, _ = ids.shape
    out = torch.full((T, cfg.H), 3.0, dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_forward_noalloc(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E,
                               gud.blob, gud.stride, gud.desc, ddv.blob, ddv.stride, ddv.desc, out)
    return out


def test_noalloc_forward_matches_workspace_forward_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = W.MoEConfig("noalloc_a", 160, 512, 256, 8, 2, 64, True, 61, zipf_s=1.1)
    small = W.MoEConfig("noalloc_b", 24, 512, 256, 8, 2, 64, True, 62)
    ids_a, w_a = W.moe_routing(big)
    ids_b, w_b = W.moe_routing(small)
    # one set of expert weights serves both calls (the small routing's experts are a subset)
    touched = set(ids_a.ravel().tolist()) | set(ids_b.ravel().tolist())
    _, _, gud, ddv, _ = moe_experts_rtn(big, touched)
    Xa, Xs = W.moe_activations(big), W.moe_activations(small)
    first = _noalloc(big, Xa, ids_a, w_a, gud, ddv)
    second = _noalloc(small, Xs, ids_b, w_b, gud, ddv)
    torch.cuda.synchronize()
    ref_a = _reference(big, Xa, ids_a, w_a, gud, ddv)
    ref_b = _reference(small, Xs, ids_b, w_b, gud, ddv)
    assert torch.equal(first.view(torch.int16), ref_a.view(torch.int16))
    assert torch.equal(second.view(torch.int16), ref_b.view(torch.int16))
    assert float(first.float().abs().max()) > 0 and float(second.float().abs().max()) > 0
