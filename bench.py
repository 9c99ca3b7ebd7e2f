"""Benchmark of the W4A8 hot path on one MI355X.

Headline (the `value`): the decode-shape fused gate/up projection, K=4096, N=14336,
symmetric INT4 g128 weights from N(0, 0.02), bf16 activations N(0, 1) with 0.1% outlier
channels x50.  One step = for M in (1, 8, 32): per-token INT8 quantization of X[M, K]
and the W4A8 GEMM (bf16 out), through w4a8_linear (one fused kernel for M <= 16).  value = weight+scale bytes streamed per step / step
time, in GB/s.  Each GEMM reads a different one of 16 device copies of the packed weights
(16 x 31.2 MB > the 256 MB Infinity Cache), so weights come from HBM.

Extra fields (same JSON line): prefill INT8 TOPS of the projection pair at M=4096
(asymmetric g128), MoE layer tokens/s of the 64-expert top-6 layer (T=512) and the
256-expert top-8 decode layer (T=64, asymmetric g64), and the pages' comparison on the
decode and prefill shapes: bf16 GEMMs through torch.mm, the W8A8 sibling (8-bit codes) and
W4A8 per-M decode times.

`roofline` is the decode GEMM at M=32 (the dominant kernel of the step): 64 back-to-back
launches on rotating weight copies between two HIP events on the launch stream;
`cpu_baseline` is the CPU oracle on the same decode step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
CALIB_BYTES = 256 << 20         # size of the calibration copy (--calib)
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, TOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200, help="timed steps (exactly this many)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=16, help="device copies of the decode weights")
    p.add_argument("--no-extra", action="store_true", help="skip the prefill and MoE figures")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--only", default="",
                   help="comma list of legs: decode,prefill,moe,quant,compare (default), moe_sparse (byte check)")
    p.add_argument("--no-graph", action="store_true", help="launch the decode steps eagerly")
    p.add_argument("--calib", action="store_true",
                   help="also run one plain copy kernel (torch.neg over 256 MiB of fp32) so that "
                        "hardware byte counters can be scaled against a known size")
    return p.parse_args()


def random_device_blobs(L, d, E, seed, dev):
    """E packed expert blobs of desc d, generated on the device: codes uniform over the
    format's range, scales |N(0, 0.02)|/7 + 1e-4, zero points in [4, 11].  The header bytes
    come from the library's packer (they are never read by the kernels)."""
    import torch
    n = L.w4a8_packed_size(d)
    G = d.K // d.group_size
    Np = (d.N + 15) // 16 * 16
    hdr = L.w4a8_pack_codes(L.desc(128, d.N, d.group_size, d.asymmetric), np.zeros((128, d.N), np.int8),
                            np.zeros((128 // d.group_size, d.N), np.float32),
                            np.zeros((128 // d.group_size, d.N), np.uint8) if d.asymmetric else None)[:256].copy()
    # patch K and the section table of the header for the real desc
    import struct
    codes_b = Np * d.K // 2
    al = lambda v: (v + 255) // 256 * 256
    so = al(256 + codes_b)
    ssz = 2 if d.scale_bits == 16 else 4                 # binary16 or float32 scales
    zo = al(so + Np * G * ssz)
    struct.pack_into("<iiiiI", hdr, 16, d.K, d.N, d.group_size, d.asymmetric, 1 if ssz == 2 else 0)
    struct.pack_into("<7Q", hdr, 40, 256, codes_b, so, Np * G * ssz, zo, Np * G if d.asymmetric else 0, n)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    buf = torch.empty(E * n, dtype=torch.uint8, device=dev)
    for e in range(E):
        b = buf[e * n:(e + 1) * n]
        b[:256].copy_(torch.from_numpy(hdr))
        if d.asymmetric:
            nib = torch.randint(0, 16, (codes_b, 2), device=dev, generator=g, dtype=torch.int16)
        else:
            nib = torch.randint(-7, 8, (codes_b, 2), device=dev, generator=g, dtype=torch.int16) & 0xF
        b[256:256 + codes_b].copy_((nib[:, 0] | (nib[:, 1] << 4)).to(torch.uint8))
        sc = (torch.randn(Np * G, device=dev, generator=g).abs() * (0.02 / 7) + 1e-4).float()
        if ssz == 2:
            sc = sc.half()
        b[so:so + Np * G * ssz].copy_(sc.view(torch.uint8))
        if d.asymmetric:
            b[zo:zo + Np * G].copy_(torch.randint(4, 12, (Np * G,), device=dev, generator=g).to(torch.uint8))
    return buf, n


class Timer:
    """HIP events on torch's current stream (the stream every launch below uses)."""

    def __init__(self, torch):
        self.t = torch
        self.pairs = []

    def start(self):
        e = self.t.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.t.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        self.t.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")


# ---------------------------------------------------------------------------------- decode
def decode_leg(args, L, W, torch, dev):
    cfg = W.C2
    d = L.desc(cfg.K, cfg.N, cfg.group_size, cfg.asymmetric)
    _, Wt = W.dense_inputs(cfg, M=1)
    host = L.w4a8_pack(d, Wt)
    n = L.w4a8_packed_size(d)
    copies = torch.empty((args.copies, n), dtype=torch.uint8, device=dev)
    one = torch.from_numpy(host).to(dev)
    for c in range(args.copies):
        copies[c].copy_(one)
    Ms = W.C2_M
    X, Xq, sx, Y = {}, {}, {}, {}
    for M in Ms:
        Xb, _ = W.dense_inputs(W.with_decode_m(cfg, M))
        X[M] = Xb.to(dev)
        Xq[M] = torch.empty((M, cfg.K), dtype=torch.int8, device=dev)
        sx[M] = torch.empty(M, dtype=torch.float32, device=dev)
        Y[M] = torch.empty((M, cfg.N), dtype=torch.bfloat16, device=dev)
    wbytes = cfg.K * cfg.N // 2 + (cfg.K // cfg.group_size) * cfg.N * 4   # codes + scales
    counter = [0]

    def step():
        for M in Ms:
            c = counter[0] % args.copies
            counter[0] += 1
            L.w4a8_linear(X[M], copies[c], d, Y[M], Xq[M], sx[M], L.W4A8_OUT_BF16)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region is exactly `steps` steps.  With graphs (the default) they are captured
    # once into one HIP graph (the weight-copy rotation continues through it, so consecutive
    # GEMMs read different copies), the graph is replayed once untimed, then once timed.
    steps = args.steps
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                step()
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / steps
    value = len(Ms) * wbytes * steps / dt / 1e9
    # the same region timed again with HIP events on the launch stream, 5 repeats: median and
    # spread of the step time (reported beside `value`)
    ev_ms = []
    if graph is not None:
        for _ in range(5):
            t = Timer(torch)
            s_ = t.start()
            graph.replay()
            t.stop(s_)
            ev_ms.append(t.mean_ms() / steps)
    # the dominant kernel (decode GEMM, M = 32): 64 back-to-back launches on rotating weight
    # copies between two HIP events on the launch stream; per-launch mean.  The launches are
    # replayed from a HIP graph so that the host's launch rate does not pace them.
    def k_launches():
        for i in range(64):
            L.w4a8_gemm(Xq[32], sx[32], copies[i % args.copies], d, Y[32], L.W4A8_OUT_BF16)

    kgraph = None
    if not args.no_graph:
        kgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(kgraph):
            k_launches()
        kgraph.replay()
        torch.cuda.synchronize()
    kt = Timer(torch)
    for rep in range(4):
        s = kt.start()
        if kgraph is not None:
            kgraph.replay()
        else:
            k_launches()
        kt.stop(s)
    kt.pairs = kt.pairs[1:]
    k_ms = kt.mean_ms() / 64
    if args.calib:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)            # reads CALIB_BYTES, writes CALIB_BYTES
        torch.cuda.synchronize()
        del src, dst
    M = 32
    kbytes = wbytes + M * cfg.K + 4 * M + 2 * M * cfg.N    # + Xq, sx, Y (bf16)
    achieved = kbytes / (k_ms * 1e-3) / 1e9
    return dict(value=value, ms_per_step=ms_step, steps=steps, weight_bytes=wbytes, kernel_ms=k_ms,
                kernel_bytes=kbytes, achieved=achieved, kernel=L.w4a8_kernel_name(d, 32), host_blob=host, Wt=Wt,
                graph=graph is not None, event_ms=ev_ms)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none or it was taken on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip().split()[0] if v.strip() else ""
    # the source file that holds the kernel (named in the summary) must be the one the counters
    # were taken on
    src = os.path.join(ROOT, "moe_token_int8_amd", "csrc", rec.get("kernel_source_file", "w4a8_kernels.hip"))
    if not os.path.exists(src) or rec.get("kernel_source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return int(rec["traffic_bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(args, leg, W):
    """The oracle on the same decode step (weights quantized once, outside the timing), with BLAS
    limited to the cores this process may run on."""
    import oracle as O
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:
        limiter = None
    cfg = W.C2
    codes, scales, zeros = O.quant_weight(leg["Wt"], cfg.group_size, cfg.asymmetric)
    xs = {M: W.bf16_values(W.dense_inputs(W.with_decode_m(cfg, M))[0]) for M in W.C2_M}

    def one_step():
        for M in W.C2_M:
            q, s = O.quant_act(xs[M])
            O.bf16_rne(O.gemm(q, s, codes, scales, zeros, cfg.group_size))

    one_step()                                        # warm-up
    n, t0 = 0, time.perf_counter()
    while True:
        one_step()
        n += 1
        if time.perf_counter() - t0 >= args.cpu_seconds or n >= 50:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": len(W.C2_M) * leg["weight_bytes"] * n / dt / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} full decode steps (quant + GEMM for M=1,8,32; K=4096, N=14336) in {dt:.1f} s; "
                      f"numpy/BLAS on {threads} threads of {cpu_model()}, weights quantized once beforehand"}


# ---------------------------------------------------------------------------------- prefill
def prefill_leg(args, L, W, torch, dev, steps):
    """The projection pair at M = 4096 (asymmetric g128), and the up projection again with
    g = 256 (half the per-group epilogues), with per-channel scales (g = K: one epilogue), with
    binary16 group scales, with g = 64 (two epilogues per superblock) and with g = 32 (four),
    the same weights otherwise."""
    out = {}
    import dataclasses
    g256 = dataclasses.replace(W.C3_UP, name=W.C3_UP.name.replace("g128", "g256"), group_size=256)
    gk = dataclasses.replace(W.C3_UP, name=W.C3_UP.name.replace("g128", "gK"), group_size=W.C3_UP.K)
    h16 = dataclasses.replace(W.C3_UP, name=W.C3_UP.name + "_fp16_scales")
    g64 = dataclasses.replace(W.C3_UP, name=W.C3_UP.name.replace("g128", "g64"), group_size=64)
    g32 = dataclasses.replace(W.C3_UP, name=W.C3_UP.name.replace("g128", "g32"), group_size=32)
    for cfg in (W.C3_UP, W.C3_DOWN, g256, gk, h16, g64, g32):
        d = L.desc(cfg.K, cfg.N, cfg.group_size, cfg.asymmetric, scale_bits=16 if cfg is h16 else 32)
        _, Wt = W.dense_inputs(cfg, M=1)
        blob = torch.from_numpy(L.w4a8_pack(d, Wt)).to(dev)
        del Wt
        X = W.random_activations(cfg.seed + 7919, cfg.M, cfg.K).to(dev)
        Xq = torch.empty((cfg.M, cfg.K), dtype=torch.int8, device=dev)
        sx = torch.empty(cfg.M, dtype=torch.float32, device=dev)
        Y = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            L.w4a8_quant_act(X, Xq, sx)
            L.w4a8_gemm(Xq, sx, blob, d, Y)
        tg, tq = Timer(torch), Timer(torch)
        for _ in range(steps):
            s = tq.start()
            L.w4a8_quant_act(X, Xq, sx)
            tq.stop(s)
            s = tg.start()
            L.w4a8_gemm(Xq, sx, blob, d, Y)
            tg.stop(s)
        g_ms, q_ms = tg.mean_ms(), tq.mean_ms()
        ops = 2.0 * cfg.M * cfg.N * cfg.K
        out[cfg.name] = dict(gemm_ms=g_ms, quant_ms=q_ms, tops=ops / (g_ms * 1e-3) / 1e12,
                             tops_with_quant=ops / ((g_ms + q_ms) * 1e-3) / 1e12,
                             frac_int8_peak=ops / (g_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                             kernel=L.w4a8_kernel_name(d, cfg.M))
        del blob, X, Xq, Y
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------------- MoE
def moe_sparse_leg(args, L, W, torch, dev, steps=3):
    """The 64-expert top-6 layer (H = 4096, I = 1408) on 16 tokens routed among experts 0..7
    only: 56 experts receive no rows, the 8 others 12 rows each (one 16-row tile, so each
    touched expert's weights are streamed exactly once per GEMM).  Run under rocprofv3 --pmc FETCH_SIZE,
    the grouped launches must read about 8 experts' weights, not 64.  Reports the bytes of the
    touched and of all experts for that comparison."""
    cfg = W.C4
    T, E8 = 16, 8
    # token t takes the 6 experts other than (t % 8) and ((t + 4) % 8): every expert gets 12 rows
    ids = np.array([[e for e in range(E8) if e not in (t % E8, (t + 4) % E8)] for t in range(T)], np.int32)
    w = np.full(ids.shape, 1.0 / cfg.topk, np.float32)
    gud = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric)
    dd = L.desc(cfg.I, cfg.H, cfg.group_size, cfg.asymmetric)
    gu, gstride = random_device_blobs(L, gud, cfg.E, 41, dev)
    dn, dstride = random_device_blobs(L, dd, cfg.E, 43, dev)
    X = W.moe_activations(cfg, T=T).to(dev)
    ids_d, w_d = torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)
    ws = torch.empty(L.w4a8_moe_workspace_size(T, cfg.topk, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=dev)
    o = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    for _ in range(steps):
        L.w4a8_moe_forward(X, ids_d, w_d, cfg.E, gu, gstride, gud, dn, dstride, dd, ws, o)
    torch.cuda.synchronize()
    touched = len(set(ids.ravel().tolist()))
    return dict(layers=steps, tokens=T, experts=cfg.E, experts_touched=touched,
                gate_up_bytes_touched=touched * gstride, down_bytes_touched=touched * dstride,
                gate_up_bytes_all=cfg.E * gstride, down_bytes_all=cfg.E * dstride)


def moe_leg(args, L, W, torch, dev, steps):
    out = {}
    for cfg, seed in ((W.C4, 4), (W.C5, 5)):
        ids, w = W.moe_routing(cfg)
        gud = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric)
        dd = L.desc(cfg.I, cfg.H, cfg.group_size, cfg.asymmetric)
        gu, gstride = random_device_blobs(L, gud, cfg.E, seed * 7, dev)
        dn, dstride = random_device_blobs(L, dd, cfg.E, seed * 11, dev)
        X = W.moe_activations(cfg).to(dev)
        ids_d = torch.from_numpy(ids).to(dev)
        w_d = torch.from_numpy(w).to(dev)
        ws = torch.empty(L.w4a8_moe_workspace_size(cfg.T, cfg.topk, cfg.H, cfg.I, cfg.E), dtype=torch.uint8,
                         device=dev)
        o = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)

        # static per-expert activation scales (values do not change the work)
        ws_st = torch.empty(L.w4a8_moe_static_workspace_size(cfg.T, cfg.topk, cfg.H, cfg.I, cfg.E),
                            dtype=torch.uint8, device=dev)
        s_gu = torch.full((cfg.E,), 0.05, dtype=torch.float32, device=dev)
        s_dn = torch.full((cfg.E,), 0.02, dtype=torch.float32, device=dev)

        def run():
            L.w4a8_moe_forward(X, ids_d, w_d, cfg.E, gu, gstride, gud, dn, dstride, dd, ws, o)

        def run_static():
            L.w4a8_moe_forward_static(X, ids_d, w_d, cfg.E, gu, gstride, gud, dn, dstride, dd, s_gu, s_dn, ws_st, o)

        def timed(fn):
            for _ in range(3):
                fn()
            t = Timer(torch)
            for _ in range(steps):
                s = t.start()
                fn()
                t.stop(s)
            return t.mean_ms()

        # the static layer as the unfused chain of entry points (the gate/up output goes through
        # HBM in bf16 and the SiLU-requant is a launch of its own), to show what the fused
        # epilogue of w4a8_moe_forward_static saves
        R = cfg.T * cfg.topk
        c_rows = torch.empty(R, dtype=torch.int32, device=dev)
        c_off = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
        c_inv = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=dev)
        c_xq = torch.empty((R, cfg.H), dtype=torch.int8, device=dev)
        c_sx = torch.empty(R, dtype=torch.float32, device=dev)
        c_gu = torch.empty((R, 2 * cfg.I), dtype=torch.bfloat16, device=dev)
        c_hq = torch.empty((R, cfg.I), dtype=torch.int8, device=dev)
        c_sh = torch.empty(R, dtype=torch.float32, device=dev)
        c_yd = torch.empty((R, cfg.H), dtype=torch.bfloat16, device=dev)

        def run_static_unfused():
            L.w4a8_moe_align(ids_d, cfg.E, c_rows, c_off, c_inv)
            L.w4a8_moe_quant_static(X, cfg.topk, c_rows, c_off, cfg.E, s_gu, c_xq, c_sx)
            L.w4a8_moe_gemm(c_xq, c_sx, None, cfg.topk, c_off, cfg.E, R, gu, gstride, gud, c_gu)
            L.w4a8_silu_mul_quant_static(c_gu, c_off, cfg.E, s_dn, c_hq, c_sh)
            L.w4a8_moe_gemm(c_hq, c_sh, None, cfg.topk, c_off, cfg.E, R, dn, dstride, dd, c_yd)
            L.w4a8_moe_combine(c_yd, c_inv, w_d, o)

        # interleaved rounds, best round per variant: no variant is favoured by when it runs
        # (clock ramp-up, what the previous variant left in the caches)
        best = {}
        for _ in range(3):
            for name, fn in (("dyn", run), ("static", run_static), ("unfused", run_static_unfused)):
                best[name] = min(best.get(name, float("inf")), timed(fn))
        ms, ms_static, ms_static_unfused = best["dyn"], best["static"], best["unfused"]
        del c_rows, c_off, c_inv, c_xq, c_sx, c_gu, c_hq, c_sh, c_yd
        # binary16 group scales: the same codes, the scales rounded to binary16 on packing
        gud16 = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric, scale_bits=16)
        dd16 = L.desc(cfg.I, cfg.H, cfg.group_size, cfg.asymmetric, scale_bits=16)
        del gu, dn
        torch.cuda.empty_cache()
        gu, gstride16 = random_device_blobs(L, gud16, cfg.E, seed * 7, dev)
        dn, dstride16 = random_device_blobs(L, dd16, cfg.E, seed * 11, dev)
        ms_h16 = timed(lambda: L.w4a8_moe_forward(X, ids_d, w_d, cfg.E, gu, gstride16, gud16, dn, dstride16, dd16,
                                                  ws, o))
        # two format classes: the first half of the experts as above (binary16 scales), the
        # second half at the other grouped-kernel group size (64 <-> 128) with float32 scales
        del gu, dn
        torch.cuda.empty_cache()
        h = cfg.E // 2
        g2 = 64 if cfg.group_size == 128 else 128
        cls = [(h, gud16, dd16), (cfg.E - h, L.desc(cfg.H, 2 * cfg.I, g2, cfg.asymmetric),
                                  L.desc(cfg.I, cfg.H, g2, cfg.asymmetric))]
        dev_sets = []
        for i, (n, gdesc, ddesc) in enumerate(cls):
            gb, gs_ = random_device_blobs(L, gdesc, n, seed * 13 + i, dev)
            db, ds_ = random_device_blobs(L, ddesc, n, seed * 17 + i, dev)
            dev_sets.append((L.DeviceWeights(gdesc, gb, gs_, n), L.DeviceWeights(ddesc, db, ds_, n)))
        ms_sets = timed(lambda: L.w4a8_moe_forward_sets(X, ids_d, w_d, dev_sets, ws, o))
        gu = dn = None
        del dev_sets
        # every expert at the second class's format (group size g2, float32 scales): with the
        # binary16-scale layer above, the two single-format layers the two-class layer mixes
        torch.cuda.empty_cache()
        gud2, dd2 = cls[1][1], cls[1][2]
        gu, gs2 = random_device_blobs(L, gud2, cfg.E, seed * 19, dev)
        dn, ds2 = random_device_blobs(L, dd2, cfg.E, seed * 23, dev)
        ms_g2 = timed(lambda: L.w4a8_moe_forward(X, ids_d, w_d, cfg.E, gu, gs2, gud2, dn, ds2, dd2, ws, o))
        del gu, dn
        gu = dn = None
        touched = len(set(ids.ravel().tolist()))
        wbytes = touched * (gstride + dstride)
        out[cfg.name] = dict(layer_ms=ms, tokens_per_s=cfg.T / (ms * 1e-3), experts_touched=touched,
                             weight_gbs=wbytes / (ms * 1e-3) / 1e9,
                             frac_hbm=wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             static_scales_layer_ms=ms_static, static_scales_unfused_chain_ms=ms_static_unfused,
                             fp16_scales_layer_ms=ms_h16,
                             two_format_classes_layer_ms=ms_sets,
                             **{f"g{g2}_scales_f32_layer_ms": ms_g2})
        del gu, dn, ws, ws_st
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------- static vs dynamic activation scales
def quant_leg(args, L, W, torch, dev, steps):
    """Per-token dynamic quantization (row abs-max reduction, then the codes) against static
    quantization with a calibrated scale (one pass), at the decode rows of the 4096-wide
    projection and at M = 4096.  Per-call means over 32 back-to-back launches replayed from a
    graph (a single launch timed alone measures the event overhead, not the kernel)."""
    out = {}
    s = torch.tensor([0.05], dtype=torch.float32, device=dev)
    per_graph = 32
    for M in (1, 8, 32, 4096):
        K = 4096
        X = W.random_activations(M, M, K).to(dev)
        Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        res = {}
        for name, fn in (("dynamic_us", lambda: L.w4a8_quant_act(X, Xq, sx)),
                         ("static_us", lambda: L.w4a8_quant_act_static(X, s, Xq, sx))):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(per_graph):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            t = Timer(torch)
            for _ in range(max(2, steps // per_graph)):
                st = t.start()
                g.replay()
                t.stop(st)
            res[name] = t.mean_ms() * 1e3 / per_graph
        out[f"m{M}_k{K}"] = res
    return out


# ------------------------------------------------------- W8A8 sibling and bf16 library baseline
def compare_leg(args, L, W, torch, dev):
    """The pages' comparison (bf16 baseline, W8A8, W4A16, W4A8) on the same shapes: bf16 GEMMs
    through torch.mm (the platform's library GEMM), the W8A8 sibling (8-bit symmetric codes,
    g = 128, the same kernels without the unpack), the W4A16 sibling (bfloat16 activations, the
    same 4-bit blob, bfloat16 MFMA) and W4A8, all measured the same way.  Decode: per-call
    means of w4a8_linear / torch.mm over 16 rotating weight copies, launches replayed from a
    graph.  Prefill: the projection pair at M = 4096, GEMM only."""
    out = {"decode": {}, "prefill": {}}
    cfg = W.C2
    K, N = cfg.K, cfg.N
    ncopy = args.copies
    d = L.desc(K, N, cfg.group_size, cfg.asymmetric)
    d8 = L.desc(K, N, cfg.group_size, False, bits=8)
    d16 = L.desc(K, N, cfg.group_size, cfg.asymmetric, scale_bits=16)
    d32 = L.desc(K, N, 32, cfg.asymmetric)
    _, Wt = W.dense_inputs(cfg, M=1)

    def copies(desc):
        one = torch.from_numpy(L.w4a8_pack(desc, Wt)).to(dev)
        t = torch.empty((ncopy, one.numel()), dtype=torch.uint8, device=dev)
        for c in range(ncopy):
            t[c].copy_(one)
        return t

    blobs, blobs8, blobs16, blobs32 = copies(d), copies(d8), copies(d16), copies(d32)
    wb = torch.from_numpy(Wt).to(dev).to(torch.bfloat16)
    Wb = torch.empty((ncopy, K, N), dtype=torch.bfloat16, device=dev)
    for c in range(ncopy):
        Wb[c].copy_(wb)
    del wb, Wt

    def per_call_us(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        t = Timer(torch)
        for _ in range(4):
            s = t.start()
            g.replay()
            t.stop(s)
        t.pairs = t.pairs[1:]
        return t.mean_ms() * 1e3 / ncopy

    for M in W.C2_M:
        Xb, _ = W.dense_inputs(W.with_decode_m(cfg, M))
        X = Xb.to(dev)
        Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def w4a8():
            for c in range(ncopy):
                L.w4a8_linear(X, blobs[c], d, Y, Xq, sx, L.W4A8_OUT_BF16)

        def w8a8():
            for c in range(ncopy):
                L.w4a8_linear(X, blobs8[c], d8, Y, Xq, sx, L.W4A8_OUT_BF16)

        def bf16():
            for c in range(ncopy):
                torch.mm(X, Wb[c], out=Y)

        def w4a8_h16():
            for c in range(ncopy):
                L.w4a8_linear(X, blobs16[c], d16, Y, Xq, sx, L.W4A8_OUT_BF16)

        def w4a8_g32():
            for c in range(ncopy):
                L.w4a8_linear(X, blobs32[c], d32, Y, Xq, sx, L.W4A8_OUT_BF16)

        def w4a16():
            for c in range(ncopy):
                L.w4a16_gemm(X, blobs[c], d, Y, L.W4A8_OUT_BF16)

        t4, t8, tb, t16 = per_call_us(w4a8), per_call_us(w8a8), per_call_us(bf16), per_call_us(w4a8_h16)
        t32 = per_call_us(w4a8_g32)
        ta16 = per_call_us(w4a16)
        out["decode"][f"m{M}"] = dict(w4a8_linear_us=t4, w8a8_linear_us=t8, bf16_mm_us=tb, w4a16_gemm_us=ta16,
                                      w4a8_fp16_scales_linear_us=t16, w4a8_g32_linear_us=t32,
                                      w4a16_kernel=L.w4a16_kernel_name(d, M),
                                      w4a8_vs_w8a8=t8 / t4, w4a8_vs_bf16=tb / t4,
                                      w8a8_weight_gbs=(K * N + K // cfg.group_size * N * 4) / (t8 * 1e-6) / 1e9,
                                      bf16_weight_gbs=K * N * 2 / (tb * 1e-6) / 1e9)
        del X, Xq, sx, Y
    del blobs, blobs8, blobs16, blobs32, Wb
    torch.cuda.empty_cache()
    for pc in (W.C3_UP, W.C3_DOWN):
        X = W.random_activations(pc.seed + 7919, pc.M, pc.K).to(dev)
        Wf = W.random_weights(pc.seed, pc.K, pc.N)
        Wm = torch.from_numpy(Wf).to(dev).to(torch.bfloat16)
        p8 = L.desc(pc.K, pc.N, pc.group_size, False, bits=8)
        blob8 = torch.from_numpy(L.w4a8_pack(p8, Wf)).to(dev)
        p4 = L.desc(pc.K, pc.N, pc.group_size, pc.asymmetric)
        blob4 = torch.from_numpy(L.w4a8_pack(p4, Wf)).to(dev)
        del Wf
        Xq = torch.empty((pc.M, pc.K), dtype=torch.int8, device=dev)
        sx = torch.empty(pc.M, dtype=torch.float32, device=dev)
        L.w4a8_quant_act(X, Xq, sx)
        Y = torch.empty((pc.M, pc.N), dtype=torch.bfloat16, device=dev)

        def timed(fn):
            for _ in range(3):
                fn()
            t = Timer(torch)
            for _ in range(10):
                s = t.start()
                fn()
                t.stop(s)
            return t.mean_ms()

        ms_b = timed(lambda: torch.mm(X, Wm, out=Y))
        ms_8 = timed(lambda: L.w4a8_gemm(Xq, sx, blob8, p8, Y))
        ms_a16 = timed(lambda: L.w4a16_gemm(X, blob4, p4, Y))
        ops = 2.0 * pc.M * pc.N * pc.K
        out["prefill"][pc.name] = dict(bf16_mm_ms=ms_b, bf16_tflops=ops / (ms_b * 1e-3) / 1e12,
                                       w8a8_gemm_ms=ms_8, w8a8_tops=ops / (ms_8 * 1e-3) / 1e12,
                                       w8a8_kernel=L.w4a8_kernel_name(p8, pc.M),
                                       w4a16_gemm_ms=ms_a16, w4a16_tflops=ops / (ms_a16 * 1e-3) / 1e12,
                                       w4a16_kernel=L.w4a16_kernel_name(p4, pc.M))
        del X, Wm, Y, Xq, sx, blob8, blob4
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_token_int8_amd as L
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    L.lib()
    legs = set(args.only.split(",")) if args.only else {"decode", "prefill", "moe", "quant", "compare"}
    if args.no_extra:
        legs = {"decode"}
    print(f"[bench] decode leg: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    leg = decode_leg(args, L, W, torch, dev)
    extra = {}
    if "prefill" in legs:
        print("[bench] prefill leg", file=sys.stderr, flush=True)
        extra["prefill"] = prefill_leg(args, L, W, torch, dev, steps=10)
    if "moe" in legs:
        print("[bench] moe leg", file=sys.stderr, flush=True)
        extra["moe"] = moe_leg(args, L, W, torch, dev, steps=20)
    if "moe_sparse" in legs:
        print("[bench] moe leg, 16 tokens over 8 of 64 experts", file=sys.stderr, flush=True)
        extra["moe_sparse"] = moe_sparse_leg(args, L, W, torch, dev)
    if "quant" in legs:
        print("[bench] quant leg", file=sys.stderr, flush=True)
        extra["quant"] = quant_leg(args, L, W, torch, dev, steps=256)
    if "compare" in legs:
        print("[bench] W8A8 sibling and bf16 library baseline", file=sys.stderr, flush=True)
        extra["compare"] = compare_leg(args, L, W, torch, dev)
    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args, leg, W)
    rec = {
        "metric": "W4A8 decode GEMM weight GB/s (M in {1,8,32}, K=4096, N=14336, quant+GEMM per step)",
        "value": round(leg["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": leg["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(leg["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode_dense_linear", "M": list(W.C2_M), "K": W.C2.K, "N": W.C2.N,
                   "group_size": W.C2.group_size, "asymmetric": False, "weight_copies": args.copies,
                   "hip_graph": leg["graph"],
                   "parallelism": "single_gpu"},
        "step_event_ms": {"median": round(float(np.median(leg["event_ms"])), 5),
                          "min": round(float(np.min(leg["event_ms"])), 5),
                          "max": round(float(np.max(leg["event_ms"])), 5)} if leg["event_ms"] else None,
        "roofline": {"bound": "hbm", "achieved": round(leg["achieved"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(leg["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(leg["kernel"]),
                     "kernel": leg["kernel"], "kernel_ms": round(leg["kernel_ms"], 5),
                     "kernel_bytes": leg["kernel_bytes"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
