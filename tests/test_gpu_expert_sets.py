"""GPU parity of a MoE layer whose experts come in format classes (P1 section 8: a group size
and format per expert), through w4a8_moe_forward_sets, against the oracle layer with per-expert
group sizes.  A grouped GEMM whose K fits the streaming kernels runs up to four sets in one
launch pair (each workgroup takes its expert's format); other GEMMs, and layers of more sets,
run one grouped launch per set."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, check_moe, sample_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _sets(cfg, touched, classes, seed, rtn):
    """classes: list of (n_experts, group_size, asymmetric, scale_bits).  Returns the device
    sets, the oracle's per-expert weights and group sizes."""
    sets, qw, gs = [], {}, []
    e0 = 0
    for n, g, asym, sbits in classes:
        dgu = L.desc(cfg.H, 2 * cfg.I, g, asym, scale_bits=sbits)
        dd = L.desc(cfg.I, cfg.H, g, asym, scale_bits=sbits)
        host_gu, host_d = {}, {}
        for e in range(e0, e0 + n):
            gs.append(g)
            if e not in touched:
                continue
            if rtn:
                Wgu, Wd = W.expert_weights(cfg, e)
                host_gu[e - e0], host_d[e - e0] = L.w4a8_pack(dgu, Wgu), L.w4a8_pack(dd, Wd)
                qw[e] = O.quant_weight(Wgu, g, asym, scale_bits=sbits) + O.quant_weight(Wd, g, asym, scale_bits=sbits)
            else:
                cg = W.random_codes(seed * 1009 + e, cfg.H, 2 * cfg.I, g, asym)
                cd = W.random_codes(seed * 2003 + e, cfg.I, cfg.H, g, asym)
                host_gu[e - e0], host_d[e - e0] = L.w4a8_pack_codes(dgu, *cg), L.w4a8_pack_codes(dd, *cd)
                r = (lambda c: (c[0], c[1].astype(np.float16).astype(np.float32), c[2])) if sbits == 16 else (lambda c: c)
                qw[e] = r(cg) + r(cd)
        sets.append((L.experts_to_device(dgu, n, host_gu), L.experts_to_device(dd, n, host_d)))
        e0 += n
    return sets, qw, gs


def _run(cfg, Xb, ids, w, sets):
    T, k = ids.shape
    ws = torch.empty(L.w4a8_moe_workspace_size(T, k, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_forward_sets(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), sets, ws, out)
    return out


@pytest.mark.parametrize("name", ["small_rtn", "small_rtn_five_classes", "c4_two_classes", "c5_4tok_two_classes",
                                  "c5_full_two_classes_sampled"])
def test_moe_forward_expert_sets(name):
    if name == "small_rtn":
        cfg, T, rtn = W.MoEConfig("small", 40, 512, 256, 8, 2, 64, True, 51), None, True
        classes = [(4, 64, True, 32), (2, 128, False, 16), (2, 128, True, 32)]
    elif name == "small_rtn_five_classes":             # more sets than one launch takes: one launch per set
        cfg, T, rtn = W.MoEConfig("small5", 40, 512, 256, 8, 2, 64, True, 53), None, True
        classes = [(2, 64, True, 32), (2, 128, False, 16), (1, 128, True, 32), (2, 64, False, 16), (1, 64, True, 16)]
    elif name == "c4_two_classes":                     # hot experts take the 128-row MFMA tiles
        cfg, T, rtn = W.C4, None, False
        classes = [(32, 128, False, 32), (32, 64, True, 16)]
    elif name == "c5_4tok_two_classes":
        cfg, T, rtn = W.C5, 4, False
        classes = [(128, 64, True, 32), (128, 128, True, 16)]
    else:                                              # full T = 64; the oracle checks 6 tokens
        cfg, T, rtn = W.C5, None, False
        classes = [(128, 64, True, 32), (128, 128, True, 16)]
    _print(f"expert sets {name}: {classes}")
    ids, w = W.moe_routing(cfg, T=T) if T else W.moe_routing(cfg)
    Xb = W.moe_activations(cfg, T=T) if T else W.moe_activations(cfg)
    tok = sample_tokens(ids.shape[0], 6, 55) if name.endswith("_sampled") else np.arange(ids.shape[0])
    sets, qw, gs = _sets(cfg, set(ids[tok].ravel().tolist()), classes, 9, rtn)
    out = _run(cfg, Xb, ids, w, sets)
    ref = O.moe_layer(W.bf16_values(Xb)[tok], ids[tok], w[tok], lambda e: qw[e], cfg.E, cfg.I, gs)
    check_moe(out[torch.from_numpy(tok).to(DEV)], ref, qw, gs)


def test_one_set_equals_moe_forward():
    """A single class is the plain layer: bit-identical to w4a8_moe_forward."""
    cfg = W.MoEConfig("one", 33, 256, 128, 16, 4, 128, True, 52)
    ids, w = W.moe_routing(cfg)
    Xb = W.moe_activations(cfg)
    sets, _, _ = _sets(cfg, set(ids.ravel().tolist()), [(16, 128, True, 32)], 3, True)
    out = _run(cfg, Xb, ids, w, sets)
    T, k = ids.shape
    ws = torch.empty(L.w4a8_moe_workspace_size(T, k, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    ref = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    gu, dn = sets[0]
    L.w4a8_moe_forward(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E,
                       gu.blob, gu.stride, gu.desc, dn.blob, dn.stride, dn.desc, ws, ref)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("asym,sbits,split", [(True, 32, (3, 5)), (False, 16, (1, 3, 2, 2))])
def test_sets_of_one_format_equal_one_set(asym, sbits, split):
    """Experts split into sets that share one format give the bits of the single-set layer: one
    launch over the sets runs each expert with the code of its own set's format, the same code
    the single-set launch runs.  The skewed routing gives some experts 128-row MFMA tiles."""
    cfg = W.MoEConfig("split", 300, 1024, 384, 8, 2, 64, asym, 61, zipf_s=1.5)
    ids, w = W.moe_routing(cfg)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    assert counts.max() >= 96, counts                  # the MFMA-tile launch has work
    _print(f"sets of one format: split {split}, rows per expert {counts.tolist()}")
    Xb = W.moe_activations(cfg)
    dgu = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, asym, scale_bits=sbits)
    dd = L.desc(cfg.I, cfg.H, cfg.group_size, asym, scale_bits=sbits)
    hgu, hd = {}, {}
    for e in range(cfg.E):
        hgu[e] = L.w4a8_pack_codes(dgu, *W.random_codes(7 * 1009 + e, cfg.H, 2 * cfg.I, cfg.group_size, asym))
        hd[e] = L.w4a8_pack_codes(dd, *W.random_codes(7 * 2003 + e, cfg.I, cfg.H, cfg.group_size, asym))
    one = [(L.experts_to_device(dgu, cfg.E, hgu), L.experts_to_device(dd, cfg.E, hd))]
    many, e0 = [], 0
    for n in split:
        many.append((L.experts_to_device(dgu, n, {e - e0: hgu[e] for e in range(e0, e0 + n)}),
                     L.experts_to_device(dd, n, {e - e0: hd[e] for e in range(e0, e0 + n)})))
        e0 += n
    ref = _run(cfg, Xb, ids, w, one)
    out = _run(cfg, Xb, ids, w, many)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
