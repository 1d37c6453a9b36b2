#!/usr/bin/env python3
"""Benchmark of the Delta-CoMe multi-tenant decode step on one MI355X.

Workload (synthetic, seeded): Llama-2-7B decoder shapes, 32 layers x 7
matrices (q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008), one
shared bf16 backbone, 50 distinct tenant deltas resident in HBM, each at the
1/16 budget (8/3/2-bit rank groups 2/32/968 or 2/47/1414), 64 decode tokens
routed to tenants by Zipf(1.1).  One step = per layer four grouped calls
(dc_apply_multitenant_group: q+k+v, o, gate+up, down): routing, activation
staging, backbone product, V side, U side and the bf16 epilogue, all on the
GPU.

Prints one JSON line.  value = tokens/s of the fused step (backbone +
delta).  The delta-only step (backbone product skipped) is timed too, as
the packed-delta bandwidth figure.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# The arithmetic of the path: 3- and 2-bit codes as fp6/fp4 matrix-core
# operands against activations in exact fp8 pieces (block-scaled MFMA), the
# 8-bit pairs on the vector ALU with fp16 weights, the backbone as bf16 MFMA;
# every sum in fp32, one bf16 rounding at the end.
DTYPE = "fp4/fp6 x fp8 mx-MFMA + bf16 MFMA, fp32 sums"
METRIC = "delta-apply tokens/s + effective packed-delta HBM GB/s (% of peak), 7B shapes"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Hip:
    """HIP events through libamdhip64 (plumbing for per-kernel timing)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(ctypes.c_void_p(e))


def spec_templates(sp, dev, torch, trs, synth):
    """Two host-packed buffers of one spec (scale/zero/sigma drawn, codes
    zero) and the mask of its valid code bits: a tenant's buffer is random
    code bits ANDed with the mask and ORed with a template."""
    import numpy as np
    out, inn, n8, n3, n2 = sp
    r = n8 + n3 + n2
    ts = []
    for k in range(2):
        d = synth.random_delta_codes(np.random.default_rng(1000 + 7 * k + out), out, inn, n8, n3, n2)
        nc = trs.dc_pack_codes(sp, np.zeros_like(d.codes_u), np.zeros_like(d.codes_v), d.sz_u, d.sz_v, d.sigma)
        ts.append(torch.from_numpy(nc).to(dev))
    widths = np.array([8] * n8 + [3] * n3 + [2] * n2)
    full = ((1 << widths) - 1).astype(np.uint8)[:, None]
    mk = trs.dc_pack_codes(sp, np.broadcast_to(full, (r, out)), np.broadcast_to(full, (r, inn)),
                           np.zeros((r, out // 128, 2), np.uint16), np.zeros((r, inn // 128, 2), np.uint16),
                           np.zeros(r, np.float32))
    return ts, torch.from_numpy(mk).to(dev)


def random_pool(nbytes, dev, torch):
    pool = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    chunk = 1 << 29
    for o in range(0, pool.numel(), chunk):
        n = min(chunk, pool.numel() - o)
        pool[o:o + n] = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    return pool


def build_c2(layers, dev, torch, trs, synth):
    """Resident deltas for every (layer, matrix, tenant) plus backbone and x."""
    n_ten, T = synth.C2_TENANTS, synth.C2_TOKENS
    mats = synth.LLAMA2_7B
    specs = [(o, i) + synth.groups_for(o, i, 16) for _, o, i in mats]
    # Per distinct spec: two host-packed templates (scale/zero/sigma) and the
    # mask of valid code bits; codes of every tenant are drawn on the GPU.
    tmpl, mask = {}, {}
    for sp in sorted(set(specs)):
        tmpl[sp], mask[sp] = spec_templates(sp, dev, torch, trs, synth)
    per_layer = sum(trs.dc_packed_bytes(sp) for sp in specs) * n_ten
    pool = random_pool(per_layer * layers, dev, torch)
    views = []
    off = 0
    for l in range(layers):
        row = []
        for m, sp in enumerate(specs):
            nb = trs.dc_packed_bytes(sp)
            vs = []
            for k in range(n_ten):
                buf = pool[off:off + nb]
                buf.bitwise_and_(mask[sp]).bitwise_or_(tmpl[sp][(k + l + m) % 2])
                vs.append(trs.DeltaView(sp, buf))
                off += nb
            row.append(vs)
        views.append(row)
    W = [[(torch.randn(o, i, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16) for _, o, i in mats]
         for _ in range(layers)]
    X = [[torch.randn(T, i, device=dev).to(torch.bfloat16).view(torch.int16) for _, o, i in mats]
         for _ in range(layers)]
    torch.cuda.synchronize()
    return specs, views, W, X, pool


def build_baselines(kind, layers, n_ten, mats, budget, dev, torch, trs, synth):
    """Resident baseline deltas for every (layer, matrix, tenant): BitDelta
    sign bits drawn uniformly on the GPU with one scale per buffer, or
    low-rank fp16 pairs drawn N(0, 1/64) on the GPU (finite values in every
    byte, padding included) with sigma_i = 0.05 i^-0.8.  Returns views
    [layer][matrix][tenant] and the pool."""
    import numpy as np
    BD = kind == trs.DC_KIND_BITDELTA
    rs = [0 if BD else synth.lowrank_r(o, i, budget) for _, o, i in mats]
    nb = [trs.dc_baseline_bytes(kind, o, i, r) for (_, o, i), r in zip(mats, rs)]
    total = sum(nb) * n_ten * layers
    if BD:
        pool = random_pool(total, dev, torch)
    else:
        pool = torch.empty(total, dtype=torch.uint8, device=dev)
        h = pool.view(torch.float16)
        chunk = 1 << 28
        for o in range(0, h.numel(), chunk):
            n = min(chunk, h.numel() - o)
            h[o:o + n] = torch.randn(n, device=dev, dtype=torch.float16) * (1.0 / 64)
    views, off = [], 0
    for l in range(layers):
        row = []
        for m, (_, o, i) in enumerate(mats):
            blk = pool[off:off + nb[m] * n_ten].view(n_ten, nb[m])
            if BD:
                a = np.abs(np.random.default_rng(5000 + 7 * l + m).lognormal(-7.0, 0.5, n_ten)).astype(np.float32)
                blk[:, :4] = torch.from_numpy(a.view(np.uint8).reshape(n_ten, 4)).to(dev)
            else:
                sg = synth.sigma_profile(rs[m])
                blk[:, :4 * rs[m]] = torch.from_numpy(sg.view(np.uint8)).to(dev)[None, :]
            row.append([trs.BaselineView(kind, o, i, rs[m], blk[k]) for k in range(n_ten)])
            off += nb[m] * n_ten
        views.append(row)
    torch.cuda.synchronize()
    return views, pool, rs


def cpu_baseline(trs, synth, budget_s=12.0):
    """The oracle (plain numpy fp64, applied from packed buffers) timed on a
    bounded sample of the same workload, extrapolated to one whole step: once
    with every host core the process may use (BLAS threads = that count) and
    once with one core (BLAS limited to one thread)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import apply as oap
    from oracle import layout
    threads = len(os.sched_getaffinity(0))
    ids = synth.c2_ids()
    touched = sorted(set(ids.tolist()))

    def run(budget):
        per_shape, sample = {}, []
        t_start = time.time()
        for mi in (0, 4, 6):                      # q (4096^2), gate (11008x4096), down (4096x11008)
            t_shape = time.time()
            _, out, inn = synth.LLAMA2_7B[mi]
            w = synth.make_c2_base(0, mi)
            x = synth.make_c2_x(0, mi)
            t0 = time.perf_counter()
            oap.apply_factored(w, x, np.zeros((0, out)), np.zeros(0), np.zeros((0, inn)))
            t_base = time.perf_counter() - t0
            times = []
            for k in touched:                     # at least two tenants, then until a third of the budget
                if len(times) >= 2 and time.time() - t_shape > budget / 3:
                    break
                d = synth.make_c2_delta(0, mi, k)
                buf = layout.pack(d.spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
                sel = np.nonzero(ids == k)[0]
                t0 = time.perf_counter()
                oap.apply_packed(d.spec, buf, None, x[sel])
                times.append(time.perf_counter() - t0)
                sample.append("%s/t%d" % (synth.LLAMA2_7B[mi][0], k))
            per_shape[mi] = (t_base, float(np.mean(times)))
        # step = 32 layers x (4 square + 2 up-proj + 1 down-proj) x (base + touched tenants)
        counts = {0: 4, 4: 2, 6: 1}
        step_s = sum(synth.C2_LAYERS * c * (per_shape[mi][0] + len(touched) * per_shape[mi][1])
                     for mi, c in counts.items())
        return synth.C2_TOKENS / step_s, sample, time.time() - t_start

    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    blas_threads = blas[0]["num_threads"] if blas else None
    with threadpool_limits(limits=threads, user_api="blas"):
        v_all, smp_all, s_all = run(budget_s)
    with threadpool_limits(limits=1, user_api="blas"):
        v_one, smp_one, s_one = run(budget_s)
    what = ("numpy fp64 oracle from packed buffers (unpack, dequant, W x + U(s*(V x))) on layer 0, matrices "
            "q, gate, down, tenants sampled per shape until about a third of the budget (%s), averaged per shape and "
            "extrapolated to 32 layers x 7 matrices x %d touched tenants + backbone")
    return {"value": v_all, "unit": "tokens/s", "cores": threads, "blas_threads": blas_threads, "kind": "oracle",
            "sample": (what % (", ".join(smp_all), len(touched))) + "; %.1f s of CPU work on %d cores" % (s_all, threads),
            "value_1core": v_one,
            "sample_1core": "the same with one core (BLAS limited to one thread): %s; %.1f s" % (
                ", ".join(smp_one), s_one)}


def counter_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed hardware-counter
    summary, scaled by its copy calibration; None when there is none for this
    kernel or its source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_bytes_decode_c2.txt")
    src = os.path.join(ROOT, "tenant_rank_serving_amd", "csrc", "k_mx.hip")
    try:
        kv = {}
        for line in open(path):
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip().split()[0] if v.strip() else ""
        if kv.get("kernel") != "k_" + kernel:
            return None
        if kv.get("source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
        return int((float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_factor"]) +
                    float(kv["write_kib_per_dispatch"]) * float(kv["write_factor"])) * 1024)
    except (OSError, KeyError, ValueError):
        return None


def profile_avg_ms(kernel):
    """Average duration of `kernel` per launch (ms) from the committed
    rocprofv3 kernel-trace summary of this step, or None when there is none
    for it or the kernel sources have changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "kernels_decode_c2_bench.txt")
    try:
        want = None
        avg = None
        for line in open(path):
            f = line.split()
            if line.startswith("source_sha256:") and len(f) > 1:
                want = f[1]
            elif f and f[0] == "k_" + kernel and len(f) >= 3:
                avg = float(f[2]) * 1e-3
        h = hashlib.sha256()
        for name in ("k_mx.hip", "kernels.hip"):
            h.update(open(os.path.join(ROOT, "tenant_rank_serving_amd", "csrc", name), "rb").read())
        return avg if want == h.hexdigest() else None
    except (OSError, ValueError):
        return None


def calibrate_copy(mib=256, reps=3):
    """A plain copy of `mib` MiB, `reps` times: under a hardware-counter run its
    per-dispatch fetch and write byte counts give the scale of the counters."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": reps}), flush=True)


def pack_bench(args):
    """Quantize + pack on the GPU (dc_pack_device): the 7 matrices of one
    Llama-2-7B layer at the 1/16 budget, fp32 singular vectors resident in
    HBM; one JSON line.  The oracle (numpy quantizer + packer) and the host C
    packer are timed on the q matrix beside it."""
    import numpy as np
    import torch

    import synth
    import tenant_rank_serving_amd as trs
    from oracle import layout, quant

    trs.lib()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    mats = []
    for name, out, inn in synth.LLAMA2_7B:
        spec = (out, inn) + tuple(synth.groups_for(out, inn, 16))
        r = sum(spec[2:])
        U = torch.randn(r, out, device=dev) * 0.02
        V = torch.randn(r, inn, device=dev) * 0.02
        sg = torch.rand(r, device=dev) + 0.5
        buf = torch.empty(trs.dc_packed_bytes(spec), dtype=torch.uint8, device=dev)
        mats.append((spec, U, sg, V, buf))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    in_bytes = sum(4 * (U.numel() + V.numel() + sg.numel()) for _, U, sg, V, _ in mats)
    out_bytes = sum(trs.dc_packed_bytes(spec) for spec, *_ in mats)

    def layer():
        for spec, U, sg, V, buf in mats:
            trs.dc_pack_device(spec, U, sg, V, buf, flag)

    for _ in range(args.warmup):
        layer()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        layer()
    e1.record()
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ms = e0.elapsed_time(e1) / args.steps
    # the q matrix on the host: the C packer and the numpy oracle
    spec, U, sg, V, buf = mats[0]
    Uh, sgh, Vh = U.cpu().numpy(), sg.cpu().numpy(), V.cpu().numpy()
    t0 = time.perf_counter()
    host = trs.dc_pack(spec, Uh, sgh, Vh)
    t_host = time.perf_counter() - t0
    assert np.array_equal(host, buf.cpu().numpy()), "device and host packers differ"
    t0 = time.perf_counter()
    cu, cv, su, sv, ss = quant.compress(Uh, sgh, Vh, *spec[2:])
    layout.pack(spec, cu, cv, su, sv, ss)
    t_orc = time.perf_counter() - t0
    share = 4 * (Uh.size + Vh.size + sgh.size) / in_bytes     # the q matrix's share of the layer's input
    achieved = (in_bytes + out_bytes) / (ms * 1e-3) / 1e9
    line = {
        "metric": "quantize+pack of a Llama-2-7B layer delta (7 matrices, 1/16 budget)", "value": round(1e3 / ms, 2),
        "unit": "layers/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "dc_pack_device on q,k,v,o 4096x4096, gate,up 11008x4096, down 4096x11008, "
                               "ranks per 1/16 budget, fp32 singular vectors in HBM"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_step": int(in_bytes + out_bytes)},
        "host_packer_layers_per_s": round(share / t_host, 3),
        "cpu_baseline": {"value": round(share / t_orc, 4), "unit": "layers/s", "cores": 1, "kind": "oracle",
                         "sample": "numpy quantizer + packer on the q matrix (%.1f s), scaled by its share of the "
                                   "layer's input bytes" % t_orc},
    }
    # the eq. 5 error table of the bit allocation for the q matrix's 4096 candidate rows (a full-rank V),
    # widths 0/2/3/8, 128 calibration samples
    from oracle import alloc
    r, inn, ncal, widths = 4096, 4096, 128, (0, 2, 3, 8)
    Vf = torch.randn(r, inn, device=dev) / 64.0
    sf = torch.rand(r, device=dev) + 0.5
    Xc = torch.randn(inn, ncal, device=dev)
    ews = torch.empty(trs.dc_error_table_workspace_bytes(r, inn, len(widths)), dtype=torch.uint8, device=dev)
    err = torch.empty((r, len(widths)), dtype=torch.float64, device=dev)
    for _ in range(args.warmup + 1):
        trs.dc_error_table(sf, Vf, Xc, widths, err, flag, ews)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        trs.dc_error_table(sf, Vf, Xc, widths, err, flag, ews)
    e1.record()
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    ms_e = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * r * len(widths) * inn * ncal
    nrow = 32
    t0 = time.perf_counter()
    alloc.error_table(sf[:nrow].double().cpu().numpy(), Vf[:nrow].cpu().numpy(), Xc.double().cpu().numpy(), widths)
    t_orc_e = time.perf_counter() - t0
    line["error_table"] = {
        "workload": "dc_error_table, %d rows x %d inputs, widths %s, %d calibration samples" % (r, inn, list(widths), ncal),
        "ms": round(ms_e, 4), "product_TFLOPs_fp32": round(flops / (ms_e * 1e-3) / 1e12, 2),
        "oracle_ms_scaled": round(t_orc_e * r / nrow * 1e3, 1),
        "oracle_sample": "alloc.error_table on %d rows (%.2f s), scaled to %d rows" % (nrow, t_orc_e, r)}
    # the SVD in front of the packer (dc_svd) on the layer's two shapes, the
    # ranks the 1/16 budget keeps; the oracle's numpy SVD on a 1024 x 1024
    # sample of the same spectrum, scaled by the cube of the size
    svd = {}
    for out, inn in ((4096, 4096), (11008, 4096)):
        r = sum(synth.groups_for(out, inn, 16))
        delta = torch.from_numpy(synth.spectral_delta(21, out, inn)).to(dev)
        Us = torch.empty((r, out), device=dev)
        ss = torch.empty((r,), device=dev)
        Vs = torch.empty((r, inn), device=dev)
        sws = torch.empty(trs.dc_svd_workspace_bytes(out, inn), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sweeps = trs.dc_svd(delta, r, Us, ss, Vs, sws)
        torch.cuda.synchronize()
        svd["%dx%d" % (out, inn)] = {"pairs": r, "ms": round((time.perf_counter() - t0) * 1e3, 1), "sweeps": sweeps}
        del sws, delta
    small = synth.spectral_delta(22, 1024, 1024).astype(np.float64)
    t0 = time.perf_counter()
    quant.svd_pairs(small)
    t_svd = time.perf_counter() - t0
    svd["oracle_ms_4096x4096_scaled"] = round(t_svd * 64 * 1e3, 1)
    svd["oracle_sample"] = "quant.svd_pairs (numpy, all host cores) on 1024 x 1024 (%.2f s), times 64" % t_svd
    svd["workload"] = ("dc_svd: fp64 Gram matrix, block Jacobi, derived vectors; synthetic deltas with "
                       "sigma_i = 0.05 i^-0.8 (host wall clock, synchronous call)")
    line["svd"] = svd
    print(json.dumps(line), flush=True)


def config_bench(args):
    """The other synthetic workloads, timed one layer at a time (eager calls
    on one stream; one JSON line per token count):
      c1  Llama-2-7B layer, one tenant, decode of 1, 8 and 64 tokens
          (dc_apply_decode), 20 layer copies cycled (569 MB of deltas);
      c3  Llama-2-13B layer, prefill of 8 tenants x 2048 tokens in contiguous
          segments (dc_apply_prefill);
      c4  Mistral-7B layer (grouped-query k, v 1024x4096) at the 1/32 budget,
          16 tenants, 128 tokens (dc_apply_multitenant), 3 copies cycled.
    Fused (backbone + delta) and delta-only; flops are 2 T r (out + in) per
    matrix for the delta and 2 T out in for the backbone.  c1 and c4 also run
    the layer as grouped calls with every layer copy captured as one HIP graph
    (key grouped_graph)."""
    import numpy as np
    import torch

    import synth
    import tenant_rank_serving_amd as trs

    trs.lib()
    dev = torch.device("cuda:0")
    w = args.workload
    if w == "c1":
        name, mats, budget, n_ten, copies, counts = "Llama-2-7B", synth.LLAMA2_7B, 16, 1, 20, (1, 8, 64)
    elif w == "c3":
        name, mats, budget, n_ten, copies = "Llama-2-13B", synth.LLAMA2_13B, 16, synth.C3_TENANTS, 1
        counts = (synth.C3_TENANTS * synth.C3_TOKENS_PER,)
    else:
        name, mats, budget, n_ten, copies = "Mistral-7B", synth.MISTRAL_7B, 32, synth.C4_TENANTS, 3
        counts = (synth.C4_TOKENS,)
    specs = [(o, i) + synth.groups_for(o, i, budget) for _, o, i in mats]
    tmpl = {sp: spec_templates(sp, dev, torch, trs, synth) for sp in sorted(set(specs))}
    nbytes = [trs.dc_packed_bytes(sp) for sp in specs]
    pool = random_pool(sum(nbytes) * n_ten * copies, dev, torch)
    views, W, off = [], [], 0
    for c in range(copies):
        row = []
        for m, sp in enumerate(specs):
            vs = []
            for k in range(n_ten):
                buf = pool[off:off + nbytes[m]]
                buf.bitwise_and_(tmpl[sp][1]).bitwise_or_(tmpl[sp][0][(k + c + m) % 2])
                vs.append(trs.DeltaView(sp, buf))
                off += nbytes[m]
            row.append(vs)
        views.append(row)
        W.append([(torch.randn(o, i, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16) for _, o, i in mats])
    tmax = max(counts)
    X = [torch.randn(tmax, i, device=dev).to(torch.bfloat16).view(torch.int16) for _, o, i in mats]
    ys = {o: torch.empty((tmax, o), dtype=torch.int16, device=dev) for _, o, _ in mats}
    op = {"c1": trs.DC_OP_DECODE, "c3": trs.DC_OP_PREFILL, "c4": trs.DC_OP_MULTITENANT}[w]
    ws = torch.empty(max(trs.dc_workspace_bytes(op, [sp] * n_ten, tmax) for sp in specs), dtype=torch.uint8,
                     device=dev)
    ids_h = synth.c4_ids() if w == "c4" else None
    ids = torch.from_numpy(ids_h).to(dev) if w == "c4" else None
    seg = np.arange(n_ten + 1, dtype=np.int32) * synth.C3_TOKENS_PER
    torch.cuda.synchronize()
    log("%s: %s layer, %d tenants, %d copies, %.2f GB of deltas resident" % (w, name, n_ten, copies, pool.numel() / 1e9))

    def call(c, m, T, fused):
        wb = W[c][m] if fused else None
        x, y = X[m][:T], ys[mats[m][1]][:T]
        if w == "c1":
            trs.dc_apply_decode(views[c][m][0], wb, x, y, ws)
        elif w == "c3":
            trs.dc_apply_prefill(views[c][m], wb, x, seg, y, ws)
        else:
            trs.dc_apply_multitenant(views[c][m], wb, x, ids, y, ws)

    def ms_per_layer(T, fused):
        for _ in range(args.warmup):
            for c in range(copies):
                for m in range(len(mats)):
                    call(c, m, T, fused)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            for c in range(copies):
                for m in range(len(mats)):
                    call(c, m, T, fused)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (args.steps * copies)

    # c1: the two baselines the pages compare with (1/16 budget), the same
    # layer copies cycled; one tenant, so every token carries id 0
    base_legs = {}
    if w == "c1" and not args.no_baselines:
        zeros = torch.zeros(tmax, dtype=torch.int32, device=dev)
        for kind, bname in ((trs.DC_KIND_BITDELTA, "bitdelta"), (trs.DC_KIND_LOWRANK, "lowrank")):
            bv, bpool, rs = build_baselines(kind, copies, 1, mats, budget, dev, torch, trs, synth)
            bws = torch.empty(max(trs.dc_baseline_workspace_bytes([bv[0][m][0]], 1, tmax) for m in range(len(mats))),
                              dtype=torch.uint8, device=dev)
            alg = sum(trs.dc_baseline_algorithmic_bytes(kind, o, i, r) for (_, o, i), r in zip(mats, rs))
            base_legs[bname] = (bv, bpool, bws, alg, rs)

    def bcall(leg, c, m, T, fused):
        bv, _, bws, _, _ = leg
        trs.dc_apply_baseline_multitenant(bv[c][m], W[c][m] if fused else None, X[m][:T], zeros[:T],
                                          ys[mats[m][1]][:T], bws)

    def ms_per_layer_with(fn, T, fused):
        for _ in range(args.warmup):
            for c in range(copies):
                for m in range(len(mats)):
                    fn(c, m, T, fused)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            for c in range(copies):
                for m in range(len(mats)):
                    fn(c, m, T, fused)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (args.steps * copies)

    # c1, c4: the layer as grouped calls (q+k+v, o, gate+up, down) on one
    # stream, all layer copies captured as one HIP graph, replayed (c1: the
    # one tenant's tokens all carry id 0)
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    ym = [torch.empty((tmax, o), dtype=torch.int16, device=dev) for _, o, _ in mats]
    gids = ids if w == "c4" else torch.zeros(tmax, dtype=torch.int32, device=dev)

    def grouped_graph_ms(T, fused):
        gstream = torch.cuda.Stream()
        gws = torch.empty(max(trs.dc_group_workspace_bytes([[specs[m]] * n_ten for m in g], len(g), T) for g in groups),
                          dtype=torch.uint8, device=dev)
        calls = [trs.GroupCall([views[c][m] for m in g], [W[c][m] for m in g] if fused else None, X[g[0]][:T],
                               gids[:T], [ym[m][:T] for m in g], gws, stream=gstream.cuda_stream)
                 for c in range(copies) for g in groups]
        with torch.cuda.stream(gstream):
            for _ in range(max(args.warmup, 1)):
                for cl in calls:
                    cl()
            torch.cuda.synchronize()
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_, stream=gstream):
                for cl in calls:
                    cl()
            g_.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(gstream)
            for _ in range(args.steps):
                g_.replay()
            e1.record(gstream)
            torch.cuda.synchronize()
        del g_
        return e0.elapsed_time(e1) / (args.steps * copies)

    touched = n_ten if ids_h is None else len(set(ids_h.tolist()))
    delta_bytes = touched * sum(trs.dc_algorithmic_bytes(sp) for sp in specs)
    base_bytes = sum(o * i * 2 for _, o, i in mats)
    for T in counts:
        rank_work = sum((sp[2] + sp[3] + sp[4]) * (sp[0] + sp[1]) for sp in specs)
        f_delta = 2.0 * T * rank_work
        f_base = 2.0 * T * base_bytes / 2
        xy = T * sum(2 * (o + i) for _, o, i in mats)
        t_f = ms_per_layer(T, True)
        t_d = ms_per_layer(T, False)
        log("%s T=%d: fused %.4f ms/layer, delta-only %.4f ms/layer" % (w, T, t_f, t_d))
        res = {
            "metric": "%s layer tokens/s (delta-apply, fused with the backbone)" % name, "value": round(T / t_f * 1e3, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(t_f, 4), "higher_is_better": True, "dtype": DTYPE, "data": "synthetic",
            "config": {"workload": {"c1": "single-tenant decode", "c3": "multi-tenant prefill, contiguous segments",
                                    "c4": "multi-tenant decode"}[w] + ", %s layer (7 matrices), 1/%d budget" % (name, budget),
                       "tenants": n_ten, "tenants_touched": touched, "tokens": T, "layer_copies_cycled": copies},
            "launch": "eager, one stream, one call per matrix",
            "fused": {"ms_per_layer": round(t_f, 4), "tokens_per_s": round(T / t_f * 1e3, 1),
                      "total_GBps": round((delta_bytes + base_bytes + xy) / (t_f * 1e-3) / 1e9, 1),
                      "matrix_TFLOPs": round((f_delta + f_base) / (t_f * 1e-3) / 1e12, 2)},
            "delta_only": {"ms_per_layer": round(t_d, 4), "tokens_per_s": round(T / t_d * 1e3, 1),
                           "packed_delta_GBps": round(delta_bytes / (t_d * 1e-3) / 1e9, 1),
                           "pct_of_hbm_peak": round(100 * delta_bytes / (t_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                           "matrix_TFLOPs": round(f_delta / (t_d * 1e-3) / 1e12, 2)},
            "bytes_per_layer": {"packed_delta": int(delta_bytes), "backbone": int(base_bytes), "x_y": int(xy)},
            "flops_per_layer": {"delta": f_delta, "backbone": f_base},
        }
        if w in ("c1", "c4"):
            gf, gd = grouped_graph_ms(T, True), grouped_graph_ms(T, False)
            log("%s T=%d grouped + graph: fused %.4f ms/layer, delta-only %.4f ms/layer" % (w, T, gf, gd))
            res["grouped_graph"] = {
                "launch": "4 grouped calls per layer (q+k+v, o, gate+up, down) on one stream, every layer copy's "
                          "calls captured as one HIP graph and replayed",
                "ms_per_layer": round(gf, 4), "tokens_per_s": round(T / gf * 1e3, 1),
                "delta_only": {"ms_per_layer": round(gd, 4),
                               "packed_delta_GBps": round(delta_bytes / (gd * 1e-3) / 1e9, 1),
                               "pct_of_hbm_peak": round(100 * delta_bytes / (gd * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}}
        if base_legs:
            res["baselines"] = {}
            for bname, leg in base_legs.items():
                bf = ms_per_layer_with(lambda c, m, T_, f, leg=leg: bcall(leg, c, m, T_, f), T, True)
                bd = ms_per_layer_with(lambda c, m, T_, f, leg=leg: bcall(leg, c, m, T_, f), T, False)
                log("%s T=%d %s: fused %.4f ms/layer, delta-only %.4f ms/layer" % (w, T, bname, bf, bd))
                res["baselines"][bname] = {
                    "ms_per_layer": round(bf, 4), "tokens_per_s": round(T / bf * 1e3, 1),
                    "delta_only": {"ms_per_layer": round(bd, 4),
                                   "packed_delta_GBps": round(leg[3] / (bd * 1e-3) / 1e9, 1),
                                   "pct_of_hbm_peak": round(100 * leg[3] / (bd * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
                    "packed_delta_bytes_per_layer": int(leg[3]),
                    "launch": "dc_apply_baseline_multitenant per matrix, every token id 0",
                    "vs_deltacome_fused": round(bf / t_f, 3), "vs_deltacome_delta_only": round(bd / t_d, 3)}
        if w == "c3":
            res["mfma_utilization_vs_2.5PF_dense_bf16"] = {
                "fused": round((f_delta + f_base) / (t_f * 1e-3) / 2.5e15, 4),
                "delta_only": round(f_delta / (t_d * 1e-3) / 2.5e15, 4)}
        print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the low-rank and BitDelta legs (c1, c2)")
    ap.add_argument("--pack", action="store_true",
                    help="time quantize+pack on the GPU (one layer's deltas) instead of the apply step")
    ap.add_argument("--workload", choices=("c2", "c1", "c3", "c4"), default="c2",
                    help="c2 (default): the multi-tenant decode step; c1, c3, c4: the other synthetic "
                         "workloads, timed per layer")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path shards by tenant with no collective, and "
              "this build runs on a single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.pack:
        pack_bench(args)
        return
    if args.workload != "c2":
        config_bench(args)
        return

    import numpy as np
    import torch

    import synth
    import tenant_rank_serving_amd as trs

    trs.lib()
    dev = torch.device("cuda:0")
    hip = Hip()
    log("building c2 workload: %d layers x 7 matrices x %d tenants" % (args.layers, synth.C2_TENANTS))
    t0 = time.time()
    specs, views, W, X, pool = build_c2(args.layers, dev, torch, trs, synth)
    ids_h = synth.c2_ids()
    ids = torch.from_numpy(ids_h).to(dev)
    touched = sorted(set(ids_h.tolist()))
    T = synth.C2_TOKENS
    log("resident deltas: %.2f GB, backbone %.2f GB, built in %.1f s" %
        (pool.numel() / 1e9, sum(w.numel() * 2 for row in W for w in row) / 1e9, time.time() - t0))
    # A decoder layer's matrices in dependency order, as grouped calls: q, k
    # and v read the same input (one call of three matrices), then o; gate
    # and up read the same input (one call of two), then down.  All calls go
    # to one non-default stream (default priority), from which one step is
    # captured as a HIP graph.
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    ws_bytes = max(trs.dc_group_workspace_bytes([[specs[m]] * synth.C2_TENANTS for m in g], len(g), T)
                   for g in groups)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ys = [torch.empty((T, sp[0]), dtype=torch.int16, device=dev) for sp in specs]

    def step_calls(fused):
        """Every call of one step, in order: (group, call)."""
        return [(g, trs.GroupCall([views[l][m] for m in g], [W[l][m] for m in g] if fused else None, X[l][g[0]],
                                  ids, [ys[m] for m in g], ws, stream=stream.cuda_stream))
                for l in range(args.layers) for g in groups]

    def layered_step(fused):
        """The step as a list of grouped calls: returns run(marks=None), which
        enqueues it; marks (one event argument per call, in order) makes every
        call record HIP events around one stage."""
        plan = step_calls(fused)

        def run(marks=None):
            for i, (_, c) in enumerate(plan):
                if marks is None:
                    c()
                else:
                    c.timed_array(marks[i])
        run.ncalls = len(plan)
        run.groups = [g for g, _ in plan]
        return run

    # bytes per step: packed deltas of the touched tenants (algorithmic), backbone
    delta_bytes = args.layers * len(touched) * sum(trs.dc_algorithmic_bytes(sp) for sp in specs)
    base_bytes = args.layers * sum(sp[0] * sp[1] * 2 for sp in specs)

    def timed_steps(run, steps, warmup, marks=None):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(steps):
            run(None if marks is None else marks[k])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # Per-stage durations: one untimed pass of the fused step, calls in
    # sequence, HIP events between the stages of every call; picks the
    # dominant kernel (largest total time).
    cl = step_calls(True)
    evs = [[hip.event() for _ in range(len(trs.STAGES) + 1)] for _ in cl]
    for (_, c), ev in zip(cl, evs):
        c.timed_array(trs.MultitenantCall.event_array(ev))
    torch.cuda.synchronize()
    stage_ms = {s: [] for s in trs.STAGES}
    for ev in evs:
        for si, s in enumerate(trs.STAGES):
            stage_ms[s].append(hip.elapsed_ms(ev[si], ev[si + 1]))
    for ev in evs:
        for e in ev:
            hip.destroy(e)
    stage_avg = {s: float(np.mean(v)) for s, v in stage_ms.items()}
    stage_tot = {s: float(np.sum(v)) for s, v in stage_ms.items()}
    log("stage averages (ms/call, calls in sequence): " + ", ".join("%s %.4f" % kv for kv in stage_avg.items()))
    heavy = ("base", "vside", "uside")
    dom = max(heavy, key=lambda s: stage_tot[s])
    dom_i = trs.STAGES.index(dom)

    def outputs():
        return [y.clone() for y in ys]

    def same_bits(a, b):
        """Outputs of the replayed graph equal the eager step's bit for bit
        (every sum is added in a fixed order)."""
        diff = sum(int((x != y).sum()) for x, y in zip(a, b))
        log("graph replay vs eager: %d differing output values" % diff)
        return diff == 0

    results, eager, dom_live, step_stats = {}, {}, {}, {}
    for mode in ("fused", "delta"):
        run = layered_step(mode == "fused")
        log("timing %s step: warmup %d, steps %d" % (mode, args.warmup, args.steps))
        # (1) the timed steps: one step captured as a HIP graph (all 128 grouped calls and
        # their kernels), replayed K times
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        ref = outputs()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        if not same_bits(ref, outputs()):
            raise RuntimeError("graph replay of the %s step differs from the eager step" % mode)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        marks[0].record()
        for k in range(args.steps):
            g.replay()
            marks[k + 1].record()
        torch.cuda.synchronize()
        results[mode] = marks[0].elapsed_time(marks[-1]) / args.steps
        per = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
        step_stats[mode] = {"median": round(per[len(per) // 2], 4), "min": round(per[0], 4),
                            "max": round(per[-1], 4)}
        del g
        # (2) the same step issued eagerly, for reference
        eager[mode] = timed_steps(run, args.steps, 1)
        # (3) instrumented steps: two HIP events per call around the dominant
        # kernel, on the stream that call runs on (they add gaps, so these steps
        # are timed apart from (1))
        ev = [[(hip.event(), hip.event()) for _ in range(run.ncalls)] for _ in range(args.steps)]
        marks = [[trs.MultitenantCall.event_array([a if i == dom_i else (b if i == dom_i + 1 else None)
                                                   for i in range(len(trs.STAGES) + 1)])
                  for a, b in step_ev] for step_ev in ev]
        timed_steps(run, args.steps, 1, marks)
        d = [hip.elapsed_ms(a, b) for step_ev in ev for a, b in step_ev if a is not None]
        dom_live[mode] = float(np.mean([x for x in d if x > 0])) if d else float("nan")
        for step_ev in ev:
            for a, b in step_ev:
                hip.destroy(a)
                hip.destroy(b)
        log("%s: %.3f ms/step (graph replay), %.3f ms/step (eager); %s kernel %.4f ms per launch "
            "(instrumented steps)" % (mode, results[mode], eager[mode], dom, dom_live[mode]))

    # Algorithmic bytes per launch of each heavy stage, averaged over calls.
    def side_bytes(sp, side):
        out, inn, n8, n3, n2 = sp
        r = n8 + n3 + n2
        n = inn if side == "v" else out
        g = (inn if side == "v" else out) // 128
        return (8 * n8 + 3 * n3 + 2 * n2) * n // 8 + r * g * 4 + (4 * r if side == "v" else 0)

    # per launch = per grouped call: the sum over the group's matrices.  The
    # V side reads x (bf16) and its tenants' V codes and scales and writes t
    # (fp32, each routed token x the tenant's ranks); the U side reads its
    # tenants' U codes and scales, t and W x (fp32, the step is fused) and
    # writes y (bf16).
    gl = [g for g, _ in cl]
    td = int((ids_h >= 0).sum())   # tokens routed to a tenant
    rank = lambda sp: sp[2] + sp[3] + sp[4]
    per_launch = {
        "vside": np.mean([sum(len(touched) * side_bytes(specs[m], "v") + td * rank(specs[m]) * 4 for m in g)
                          + T * specs[g[0]][1] * 2 for g in gl]),
        "uside": np.mean([sum(len(touched) * side_bytes(specs[m], "u") + td * rank(specs[m]) * 4
                              + T * specs[m][0] * (4 + 2) for m in g) for g in gl]),
        "base": np.mean([sum(specs[m][0] * specs[m][1] * 2 for m in g) + T * specs[g[0]][1] * 2 for g in gl]),
    }
    # dom_live: the kernel's average duration per launch inside the
    # instrumented fused steps, measured with HIP events on each call's stream
    achieved = per_launch[dom] / (dom_live["fused"] * 1e-3) / 1e9
    # the same kernel's average duration per launch in the committed
    # rocprofv3 kernel trace of this step (all its launches)
    prof_ms = profile_avg_ms(dom)
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(dom),
            "bytes_per_launch": int(per_launch[dom]), "avg_launch_ms": round(dom_live["fused"], 5),
            "frac_profile": (round(per_launch[dom] / (prof_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                             if prof_ms else None),
            "avg_launch_ms_profile": prof_ms,
            "avg_launch_ms_in_sequence": round(stage_avg[dom], 5),
            "stages_avg_ms_in_sequence": {s: round(v, 5) for s, v in stage_avg.items()}}

    ms = results["fused"]
    ms_d = results["delta"]
    out = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": "multi-tenant decode, Llama-2-7B shapes: %d layers x 7 matrices, 50 resident "
                               "1/16 deltas (8/3/2-bit), shared bf16 backbone, 64 tokens Zipf(1.1)" % args.layers,
                   "layers": args.layers, "tenants_resident": synth.C2_TENANTS, "tenants_touched": len(touched),
                   "tokens": T, "step": "fused"},
        "packed_delta_GBps": round(delta_bytes / (ms * 1e-3) / 1e9, 1),
        "fused_total_GBps": round((delta_bytes + base_bytes) / (ms * 1e-3) / 1e9, 1),
        "launch": "HIP graph replay of one captured step: 128 grouped calls (q+k+v, o, gate+up, down per layer)",
        "step_ms_per_replay": step_stats,
        "eager_ms_per_step": {"fused": round(eager["fused"], 4), "delta": round(eager["delta"], 4)},
        "delta_only": {"ms_per_step": round(ms_d, 4), "tokens_per_s": round(T / (ms_d * 1e-3), 1),
                       "packed_delta_GBps": round(delta_bytes / (ms_d * 1e-3) / 1e9, 1),
                       "pct_of_hbm_peak": round(100 * delta_bytes / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
        "roofline": roof,
    }
    if not args.no_baselines:
        # The two baselines the pages compare with (1/16 budget), through the
        # same step structure: grouped calls, one captured graph per step.
        del views, pool, cl, run
        torch.cuda.empty_cache()
        out["baselines"] = {}
        for kind, name in ((trs.DC_KIND_BITDELTA, "bitdelta"), (trs.DC_KIND_LOWRANK, "lowrank")):
            t0 = time.time()
            bv, bpool, rs = build_baselines(kind, args.layers, synth.C2_TENANTS, synth.LLAMA2_7B, 16, dev, torch,
                                            trs, synth)
            log("%s: %.2f GB resident, built in %.1f s" % (name, bpool.numel() / 1e9, time.time() - t0))
            bws = torch.empty(max(trs.dc_baseline_workspace_bytes([[bv[0][m][0]] * synth.C2_TENANTS for m in g],
                                                                  len(g), T) for g in groups),
                              dtype=torch.uint8, device=dev)
            leg = {}
            for mode in ("fused", "delta"):
                calls = [trs.BaselineGroupCall([bv[l][m] for m in g], [W[l][m] for m in g] if mode == "fused"
                                               else None, X[l][g[0]], ids, [ys[m] for m in g], bws,
                                               stream=stream.cuda_stream)
                         for l in range(args.layers) for g in groups]

                def brun(marks=None, calls=calls):
                    for c in calls:
                        c()
                for _ in range(args.warmup):
                    brun()
                torch.cuda.synchronize()
                ref = outputs()
                g_ = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g_, stream=stream):
                    brun()
                for _ in range(args.warmup):
                    g_.replay()
                torch.cuda.synchronize()
                if not same_bits(ref, outputs()):
                    raise RuntimeError("graph replay of the %s %s step differs from the eager step" % (name, mode))
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    g_.replay()
                e1.record()
                torch.cuda.synchronize()
                leg[mode] = e0.elapsed_time(e1) / args.steps
                del g_
            alg = args.layers * len(touched) * sum(trs.dc_baseline_algorithmic_bytes(kind, o, i, r)
                                                   for (_, o, i), r in zip(synth.LLAMA2_7B, rs))
            out["baselines"][name] = {
                "ms_per_step": round(leg["fused"], 4), "tokens_per_s": round(T / (leg["fused"] * 1e-3), 1),
                "delta_only": {"ms_per_step": round(leg["delta"], 4),
                               "tokens_per_s": round(T / (leg["delta"] * 1e-3), 1),
                               "packed_delta_GBps": round(alg / (leg["delta"] * 1e-3) / 1e9, 1),
                               "pct_of_hbm_peak": round(100 * alg / (leg["delta"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
                "packed_delta_bytes_per_step": int(alg),
                "form": ("1 sign bit per delta entry + one fp32 scale per matrix" if kind == trs.DC_KIND_BITDELTA
                         else "fp16 top-r pairs, r = %s (q,k,v,o / gate,up / down)" % sorted(set(rs))),
                "vs_deltacome_fused": round(leg["fused"] / ms, 3),
                "vs_deltacome_delta_only": round(leg["delta"] / ms_d, 3)}
            log("%s: fused %.3f ms/step, delta-only %.3f ms/step" % (name, leg["fused"], leg["delta"]))
            del bv, bpool, bws
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(trs, synth, budget_s=8.0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
