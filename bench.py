#!/usr/bin/env python3
"""Benchmark of the fused dequantize-and-multiply path on one MI355X.

One step = one pass of the decode workload: the three q4_0 GEMVs of a Llama-7B
layer's shapes (4096x4096, 11008x4096, 4096x11008), batch 1, fp32 activations.
Inputs are seeded synthetic planes, uploaded before timing; every step reads a
different copy from a rotating pool of >= 1 GiB so that the 256 MB Infinity Cache
cannot serve repeated reads (the weights come from HBM, as in decode).

Prints ONE JSON line: value = algorithmic bytes (packed weights + scales + x + y)
per step / time per step, in GB/s.  `roofline` covers the dominant kernel, timed
with HIP events on the stream it runs on; `cpu_baseline` times the CPU oracle on
a bounded sample of the same workload.  `secondary` carries the other workloads
(q6_K GEMV, 4-bit codebook MoE, 2-bit and 3-bit additive GEMVs, 8-bit codebook GEMV,
q6_K prefill GEMM) when they run.
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

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS
POOL_BYTES = 1 << 30           # rotating pool: 4x the 256 MB Infinity Cache

METRIC = "quantized GEMV HBM GB/s (% of peak); q6_K prefill GEMM int8 TOPS (% of peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only-primary", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--secondary", default="q6_K_gemv,q6_K_decode,q4_0_batch,q4_0_q8,batch4_other,batch8_other,cb4_moe,aq2x8,aq3x8,cb8,q6_K_gemm",
                    help="comma-separated secondary workloads to run")
    return ap.parse_args()


def dev_planes(planes: dict):
    import torch
    out = {}
    for name, a in planes.items():
        a = np.ascontiguousarray(a)
        if a.dtype == np.float16:
            out[name] = torch.from_numpy(a.view(np.uint16).copy()).view(torch.float16).cuda()
        else:
            out[name] = torch.from_numpy(a.copy()).cuda()
    return out


def make_pool(qmv, fmt, n, k, seed, copies):
    """`copies` distinct device copies of one generated matrix: each plane is one
    [copies, ...] tensor filled by device-side copies, and copy c is its slice c."""
    import torch
    host = synth.gen_weights(fmt, n, k, seed=seed)
    first = dev_planes(host)
    big = {name: torch.empty((copies, *t.shape), dtype=t.dtype, device="cuda") for name, t in first.items()}
    for name, t in first.items():
        big[name][:] = t
    pool = [qmv.QWeights(fmt, n, k, {name: big[name][c] for name in big}) for c in range(copies)]
    pool[0]._keep = big
    return host, pool


def pool_copies(bytes_per_copy):
    return max(2, -(-POOL_BYTES // bytes_per_copy))


def graph_of(fn, count):
    """A HIP graph (torch.cuda.CUDAGraph) that replays fn(0) .. fn(count-1) back to back.

    The library enqueues plain kernel launches on the current stream, so stream capture
    records them; replaying the graph removes the per-launch host overhead of Python."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(min(count, 3)):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(g, count):
    """Milliseconds per item of one replay of graph g holding `count` items (HIP events
    recorded on the stream the graph replays on)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / count


def q4_0_workload(qmv, steps, warmup):
    import torch
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]
    per_set = sum(qmv.weight_bytes(synth.FMT_Q4_0, n, k) for n, k in shapes)
    copies = max(2, -(-POOL_BYTES // per_set))
    mats, xs, ys, algo = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        _, pool = make_pool(qmv, synth.FMT_Q4_0, n, k, seed=i, copies=copies)
        mats.append(pool)
        xs.append(torch.from_numpy(synth.gen_x(1, k, seed=i)).cuda())
        ys.append(torch.empty((1, n), dtype=torch.float32, device="cuda"))
        algo.append(qmv.weight_bytes(synth.FMT_Q4_0, n, k) + 4 * k + 4 * n)

    def step(i):
        c = i % copies
        for s in range(len(shapes)):
            qmv.gemv(mats[s][c], xs[s], ys[s])

    # warm-up steps, then exactly `steps` timed steps, each set captured in one graph
    gw = graph_of(lambda i: step(i + 1000), max(1, warmup))
    gt = graph_of(step, steps)
    gw.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    gt.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    bytes_step = sum(algo)
    per_shape = []
    for s, (n, k) in enumerate(shapes):
        R = max(steps, 60)
        g = graph_of(lambda i, s=s: qmv.gemv(mats[s][i % copies], xs[s], ys[s]), R)
        avg = time_graph(g, R)
        # contrast only: the same launches on one copy, which stays in the Infinity Cache
        warm = time_graph(graph_of(lambda i, s=s: qmv.gemv(mats[s][0], xs[s], ys[s]), R), R)
        qmv.gemv(mats[s][0], xs[s], ys[s])
        per_shape.append({"shape": f"{n}x{k}", "bytes": algo[s], "avg_launch_ms": avg,
                          "GBps": algo[s] / avg / 1e6, "frac": algo[s] / avg / 1e6 / HBM_PEAK_GBS,
                          "warm_one_copy_GBps": round(algo[s] / warm / 1e6, 1),
                          "path": qmv.last_path()})
    torch.cuda.synchronize()
    return {"ms_per_step": ms, "bytes_per_step": bytes_step, "GBps": bytes_step / ms / 1e6,
            "copies": copies, "pool_bytes": copies * per_set, "shapes": per_shape}


def read_ceiling(qmv, sizes, steps, large=True):
    """The stream-read ceiling: the library's read-only kernel over a rotating pool of
    distinct buffers of each size (cold, as the GEMVs' pools), and once over 4 GiB."""
    import torch
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = []
    for b in sizes:
        b16 = (b + 15) // 16 * 16
        copies = pool_copies(b16)
        pool = torch.zeros((copies, b16), dtype=torch.uint8, device="cuda")
        R = max(steps, 60)
        avg = time_graph(graph_of(lambda i: qmv.read_ceiling(pool[i % copies], sink), R), R)
        out.append({"bytes": b16, "avg_launch_ms": round(avg, 5), "GBps": round(b16 / avg / 1e6, 1)})
        del pool
    if not large:
        return {"kernel": "read_ceiling_kernel (128-bit nontemporal loads only)", "sizes": out}
    big = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    avg = time_graph(graph_of(lambda i: qmv.read_ceiling(big, sink), 5), 5)
    large = {"bytes": big.numel(), "avg_launch_ms": round(avg, 4), "GBps": round(big.numel() / avg / 1e6, 1)}
    del big
    torch.cuda.synchronize()
    return {"kernel": "read_ceiling_kernel (128-bit nontemporal loads only)", "sizes": out, "large": large}


def gemv_workload(qmv, fmt, shapes, batch, xt, steps, label):
    """Batch-`batch` GEMVs over `shapes` (one step = one GEMV per shape), rotating pool."""
    import torch
    per_set = sum(qmv.weight_bytes(fmt, n, k) for n, k in shapes)
    copies = pool_copies(per_set)
    mats, xs, ys, algo = [], [], [], []
    xbytes = 4 if xt == synth.DT_F32 else 2
    for i, (n, k) in enumerate(shapes):
        _, pool = make_pool(qmv, fmt, n, k, seed=i, copies=copies)
        mats.append(pool)
        x = synth.gen_x(batch, k, xt, seed=i)
        xd = torch.from_numpy(x).cuda() if xt == synth.DT_F32 else \
            torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        xs.append(xd)
        ys.append(torch.empty((batch, n), dtype=torch.float32, device="cuda"))
        algo.append(qmv.weight_bytes(fmt, n, k) + xbytes * batch * k + 4 * batch * n)

    def step(i):
        for s in range(len(shapes)):
            qmv.gemv(mats[s][i % copies], xs[s], ys[s])

    g = graph_of(step, steps)
    ms = time_graph(g, steps)
    per_shape = []
    for s, (n, k) in enumerate(shapes):
        R = max(steps, 40)
        avg = time_graph(graph_of(lambda i, s=s: qmv.gemv(mats[s][i % copies], xs[s], ys[s]), R), R)
        qmv.gemv(mats[s][0], xs[s], ys[s])
        per_shape.append({"shape": f"{n}x{k}", "bytes": algo[s], "avg_launch_ms": round(avg, 5),
                          "GBps": round(algo[s] / avg / 1e6, 1), "path": qmv.last_path()})
    path = qmv.last_path()
    add_ceiling(qmv, per_shape, steps)
    gbs = sum(algo) / ms / 1e6
    return {"workload": label, "value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "ms_per_step": round(ms, 5), "bytes_per_step": sum(algo), "pool_copies": copies,
            "path": path, "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
            "shapes": per_shape}


def q8_workload(qmv, fmt, batch, steps, label):
    """The GEMV over per-32 int8 activations (q4_0 or q6_K) on the three decode shapes (one
    step = one GEMV per shape, activations quantized beforehand, as they are once per
    activation vector for every GEMV that reads it).  The same step with one quantizer
    launch in front of each GEMV is timed too and reported beside it."""
    import torch
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]
    per_set = sum(qmv.weight_bytes(fmt, n, k) for n, k in shapes)
    copies = pool_copies(per_set)
    mats, xs, qs, ys, algo = [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        _, pool = make_pool(qmv, fmt, n, k, seed=i, copies=copies)
        mats.append(pool)
        x = torch.from_numpy(synth.gen_x(batch, k, synth.DT_F32, seed=i)).cuda()
        xs.append(x)
        qs.append(qmv.quant_act(x))
        ys.append(torch.empty((batch, n), dtype=torch.float32, device="cuda"))
        # weights + int8 activations and their scales + outputs
        algo.append(qmv.weight_bytes(fmt, n, k) + batch * (k + k // 8) + 4 * batch * n)

    def step(i):
        for s in range(len(shapes)):
            qmv.gemv_q8(mats[s][i % copies], qs[s][0], qs[s][1], ys[s])

    def step_quant(i):
        for s in range(len(shapes)):
            qmv.quant_act(xs[s], qs[s][0], qs[s][1])
            qmv.gemv_q8(mats[s][i % copies], qs[s][0], qs[s][1], ys[s])

    ms = time_graph(graph_of(step, steps), steps)
    ms_q = time_graph(graph_of(step_quant, steps), steps)
    per_shape = []
    for s, (n, k) in enumerate(shapes):
        R = max(steps, 40)
        avg = time_graph(graph_of(lambda i, s=s: qmv.gemv_q8(mats[s][i % copies], qs[s][0], qs[s][1], ys[s]), R), R)
        qmv.gemv_q8(mats[s][0], qs[s][0], qs[s][1], ys[s])
        per_shape.append({"shape": f"{n}x{k}", "bytes": algo[s], "avg_launch_ms": round(avg, 5),
                          "GBps": round(algo[s] / avg / 1e6, 1), "path": qmv.last_path()})
    path = qmv.last_path()
    add_ceiling(qmv, per_shape, steps)
    gbs = sum(algo) / ms / 1e6
    return {"workload": label, "value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "ms_per_step": round(ms, 5), "bytes_per_step": sum(algo), "pool_copies": copies,
            "with_quant_act": {"ms_per_step": round(ms_q, 5), "GBps": round(sum(algo) / ms_q / 1e6, 1)},
            "path": path, "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
            "shapes": per_shape}


def add_ceiling(qmv, per_shape, steps):
    """Per shape: the stream-read ceiling for its bytes and the kernel's fraction of it."""
    rc = read_ceiling(qmv, [sh["bytes"] for sh in per_shape], steps, large=False)
    for sh, c in zip(per_shape, rc["sizes"]):
        sh["read_ceiling_ms"] = c["avg_launch_ms"]
        sh["frac_of_read_ceiling"] = round(c["avg_launch_ms"] / sh["avg_launch_ms"], 4)


def moe_workload(qmv, tokens, label):
    """Routed-expert FFN, batch 1: 256 experts of gate/up 2048x7168 and down 7168x2048
    (4-bit codebook, one 16-entry fp16 codebook per 128 weights), top-8 per token.
    The 8.46 GB expert set is resident; its bytes are drawn on the device with a seeded
    generator (throughput does not depend on the values; parity is tested elsewhere)."""
    import torch
    E, dm, dff = 256, 7168, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)

    def planes(n, k):
        idx = torch.randint(0, 256, (E, n, k // 2), dtype=torch.uint8, device="cuda", generator=gen)
        cb = torch.randn((E, n, k // 128, 16), device="cuda", generator=gen) * 0.02
        cb = torch.sort(cb, dim=-1).values.to(torch.float16)
        return {"idx": idx, "cb": cb}

    G = qmv.QWeights(qmv.CB4, dff, dm, planes(dff, dm))
    U = qmv.QWeights(qmv.CB4, dff, dm, planes(dff, dm))
    D = qmv.QWeights(qmv.CB4, dm, dff, planes(dm, dff))
    ids = torch.from_numpy(synth.gen_moe_ids(tokens, E, 8, seed=0)).cuda()
    x = torch.from_numpy(synth.gen_x(tokens, dm, synth.DT_BF16, seed=0).view(np.int16).copy()).view(torch.bfloat16).cuda()
    h = torch.empty((8, dff), dtype=torch.float32, device="cuda")
    y = torch.empty((8, dm), dtype=torch.float32, device="cuda")
    per_tok = 8 * (qmv.weight_bytes(qmv.CB4, dff, dm) * 2 + qmv.weight_bytes(qmv.CB4, dm, dff)) + 2 * dm + \
        8 * dff * 4 * 2 + 8 * dm * 4

    def step(i):
        qmv.moe_ffn(G, U, D, E, ids[i % tokens], x[i % tokens], h, y)

    g = graph_of(step, tokens)
    ms = time_graph(g, tokens)
    gbs = per_tok / ms / 1e6
    return {"workload": label, "value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "ms_per_token": round(ms, 5), "bytes_per_token": per_tok, "tokens": tokens,
            "path": qmv.last_path(), "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"}}


def gemm_workload(qmv, steps, label):
    """q6_K prefill GEMM, M = 512 tokens, W 11008x4096 and 4096x11008: TOPS = 2 M N K / time
    for the int8 contraction alone (activations already quantized) and end to end.  The
    weights are registered with their pre-expanded planes (the default-on registration the
    method describes), and the in-kernel expansion of the same calls is timed beside it."""
    import torch
    M = 512
    out = {"workload": label, "unit": "TOPS", "shapes": []}
    tot_ops, tot_ms, tot_ms_e2e, tot_ms_raw = 0, 0.0, 0.0, 0.0
    for i, (n, k) in enumerate([(11008, 4096), (4096, 11008)]):
        _, pool = make_pool(qmv, synth.FMT_Q6_K, n, k, seed=i, copies=4)
        x = torch.from_numpy(synth.gen_x(M, k, seed=i)).cuda()
        xq, xs = qmv.quant_act(x)
        y = torch.empty((M, n), dtype=torch.float32, device="cuda")
        ws = torch.empty(qmv.workspace_bytes(pool[0], M), dtype=torch.uint8, device="cuda")
        R = max(8, steps // 4)
        ms_raw = time_graph(graph_of(lambda j: qmv.gemm_q8(pool[j % 4], xq, xs, y), R), R)
        path_raw = qmv.last_path()
        for W in pool:
            qmv.register_plane(W)
        ms = time_graph(graph_of(lambda j: qmv.gemm_q8(pool[j % 4], xq, xs, y), R), R)
        path = qmv.last_path()
        ms2 = time_graph(graph_of(lambda j: qmv.gemm(pool[j % 4], x, y, ws), R), R)
        for W in pool:
            qmv.unregister_plane(W)
        ops = 2 * M * n * k
        tot_ops += ops
        tot_ms += ms
        tot_ms_e2e += ms2
        tot_ms_raw += ms_raw
        out["shapes"].append({"shape": f"{n}x{k}", "M": M, "ms": round(ms, 5), "TOPS": round(ops / ms / 1e9, 1),
                              "ms_with_quantizer": round(ms2, 5), "path": path,
                              "ms_in_kernel_expand": round(ms_raw, 5),
                              "TOPS_in_kernel_expand": round(ops / ms_raw / 1e9, 1), "path_in_kernel_expand": path_raw})
    tops = tot_ops / tot_ms / 1e9
    out.update({"value": round(tops, 1), "frac_of_peak": round(tops / INT8_PEAK_TOPS, 4),
                "TOPS_with_quantizer": round(tot_ops / tot_ms_e2e / 1e9, 1),
                "TOPS_in_kernel_expand": round(tot_ops / tot_ms_raw / 1e9, 1),
                "roofline": {"bound": "mfma", "peak": INT8_PEAK_TOPS, "unit": "TOPS"}})
    return out


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed PMC record, or None
    when the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "q4_0_gemv_4096x11008_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])).hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    return rec["traffic_bytes_per_launch"] if h == rec["sources_sha256"] else None


def cpu_baseline(seconds):
    """The oracle on the same three matrices (all rows), repeated until `seconds` of work."""
    import oracle
    nth = max(1, min(16, os.cpu_count() or 1))
    shapes = [(4096, 4096), (11008, 4096), (4096, 11008)]
    mats, xs, nbytes = [], [], 0
    for i, (n, k) in enumerate(shapes):
        mats.append(oracle.Mat(synth.FMT_Q4_0, n, k, synth.gen_weights(synth.FMT_Q4_0, n, k, seed=i)))
        xs.append(synth.gen_x(1, k, seed=i))
        nbytes += (n * k // 32) * 18 + 4 * k + 4 * n
    done, t0 = 0, time.perf_counter()
    while True:
        for m, x in zip(mats, xs):
            oracle.gemv(m, x, oracle.F32, nthreads=nth)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": nbytes * done / el / 1e9, "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": f"{done} full pass(es) of the three q4_0 GEMVs (all rows), fp64 oracle, "
                      f"{el:.1f} s, OpenMP over rows"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                          "(the path shards by output rows across GPUs, not measured here)"}))
        sys.exit(2)
    import torch
    import bit_weight_quantized_dequant_amd as qmv
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    qmv.lib()
    if a.copy_ref:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    prim = q4_0_workload(qmv, a.steps, a.warmup)
    dom = max(prim["shapes"], key=lambda s: s["avg_launch_ms"])
    out = {
        "metric": METRIC,
        "value": round(prim["GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(prim["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "q4_0 GEMV batch 1, Llama-7B decode shapes 4096x4096 + 11008x4096 + "
                               "4096x11008, fp32 x, rotating HBM pool",
                   "batch": 1, "pool_bytes": prim["pool_bytes"], "pool_copies": prim["copies"],
                   "bytes_per_step": prim["bytes_per_step"]},
        "frac_of_peak": round(prim["GBps"] / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": f"q4_0 GEMV {dom['shape']} ({dom['path']})",
                     "achieved": round(dom["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom["frac"], 4),
                     "traffic": recorded_traffic() if dom["shape"] == "4096x11008" else None},
        "shapes": prim["shapes"],
    }
    if not a.only_primary:
        # the plain-read floor for each primary shape's bytes, same pool protocol
        rc = read_ceiling(qmv, [sh["bytes"] for sh in prim["shapes"]], a.steps)
        for sh, c in zip(out["shapes"], rc["sizes"]):
            sh["read_ceiling_ms"] = c["avg_launch_ms"]
            sh["frac_of_read_ceiling"] = round(c["avg_launch_ms"] / sh["avg_launch_ms"], 4)
        out["read_ceiling"] = rc
        sec = {}
        want = set(a.secondary.split(","))
        if "q6_K_gemv" in want:
            sec["q6_K_gemv"] = gemv_workload(qmv, synth.FMT_Q6_K, [(256, 1024)], 1, synth.DT_F32, 200,
                                             "q6_K GEMV batch 1, 256x1024, fp32 x")
        for b in ((2, 4, 8) if "q4_0_batch" in want else ()):
            sec[f"q4_0_gemv_b{b}"] = gemv_workload(qmv, synth.FMT_Q4_0, [(4096, 4096), (11008, 4096), (4096, 11008)],
                                                   b, synth.DT_F32, 50,
                                                   f"q4_0 GEMV batch {b}, Llama-7B decode shapes, fp32 x")
        for b in ((1, 4) if "q4_0_q8" in want else ()):
            sec[f"q4_0_q8_gemv_b{b}"] = q8_workload(
                qmv, synth.FMT_Q4_0, b, 50, f"q4_0 GEMV over per-32 int8 activations, batch {b}, Llama-7B decode shapes")
        if "q6_K_decode" in want:
            sec["q6_K_gemv_llama"] = gemv_workload(qmv, synth.FMT_Q6_K, [(4096, 4096), (11008, 4096), (4096, 11008)],
                                                   1, synth.DT_F32, 50,
                                                   "q6_K GEMV batch 1, Llama-7B decode shapes, fp32 x")
        for b in ((1, 4) if "q6_K_decode" in want else ()):
            sec[f"q6_K_q8_gemv_b{b}"] = q8_workload(
                qmv, synth.FMT_Q6_K, b, 50, f"q6_K GEMV over per-32 int8 activations, batch {b}, Llama-7B decode shapes")
        if "batch4_other" in want:
            # batch 4 for the formats the other batch lines do not cover
            sec["q6_K_gemv_b4"] = gemv_workload(qmv, synth.FMT_Q6_K, [(4096, 4096), (11008, 4096), (4096, 11008)],
                                                4, synth.DT_F32, 50, "q6_K GEMV batch 4, Llama-7B decode shapes, fp32 x")
            sec["cb4_gemv_b4"] = gemv_workload(qmv, synth.FMT_CB4, [(2048, 7168), (7168, 2048)], 4, synth.DT_BF16, 50,
                                               "4-bit codebook GEMV batch 4, 2048x7168 + 7168x2048, bf16 x")
            sec["cb8_gemv_b4"] = gemv_workload(qmv, synth.FMT_CB8, [(2048, 7168), (7168, 2048)], 4, synth.DT_BF16, 50,
                                               "8-bit codebook GEMV batch 4, 2048x7168 + 7168x2048, bf16 x")
        if "batch8_other" in want:
            # batch 8 for the formats the q4_0 batch lines do not cover
            sec["q6_K_gemv_b8"] = gemv_workload(qmv, synth.FMT_Q6_K, [(4096, 4096), (11008, 4096), (4096, 11008)],
                                                8, synth.DT_F32, 50, "q6_K GEMV batch 8, Llama-7B decode shapes, fp32 x")
            sec["cb4_gemv_b8"] = gemv_workload(qmv, synth.FMT_CB4, [(2048, 7168), (7168, 2048)], 8, synth.DT_BF16, 50,
                                               "4-bit codebook GEMV batch 8, 2048x7168 + 7168x2048, bf16 x")
            sec["cb8_gemv_b8"] = gemv_workload(qmv, synth.FMT_CB8, [(2048, 7168), (7168, 2048)], 8, synth.DT_BF16, 50,
                                               "8-bit codebook GEMV batch 8, 2048x7168 + 7168x2048, bf16 x")
            sec["aq2x8_gemv_b8"] = gemv_workload(qmv, synth.FMT_AQ2X8, [(14336, 4096), (4096, 14336)], 8,
                                                 synth.DT_BF16, 50, "2-bit additive GEMV batch 8, 14336x4096 + 4096x14336, bf16 x")
        if "cb4_moe" in want:
            sec["cb4_moe"] = moe_workload(qmv, 64, "4-bit codebook MoE FFN, batch 1, 256 experts top-8, "
                                                   "gate/up 2048x7168 + down 7168x2048, bf16 x")
        for b in ((1, 4) if "aq2x8" in want else ()):
            sec[f"aq2x8_gemv_b{b}"] = gemv_workload(qmv, synth.FMT_AQ2X8, [(14336, 4096), (4096, 14336)], b,
                                                    synth.DT_BF16, 50,
                                                    f"2-bit additive GEMV batch {b}, 14336x4096 + 4096x14336, bf16 x")
        for b in ((1, 4) if "aq3x8" in want else ()):
            sec[f"aq3x8_gemv_b{b}"] = gemv_workload(qmv, synth.FMT_AQ3X8, [(14336, 4096), (4096, 14336)], b,
                                                    synth.DT_BF16, 50,
                                                    f"3-bit additive GEMV batch {b}, 14336x4096 + 4096x14336, bf16 x")
        if "cb8" in want:
            sec["cb8_gemv"] = gemv_workload(qmv, synth.FMT_CB8, [(2048, 7168), (2048, 7168), (7168, 2048),
                                                                 (129280, 7168)], 1, synth.DT_BF16, 20,
                                            "8-bit codebook GEMV batch 1, shared expert gate/up 2048x7168 + "
                                            "down 7168x2048 and output head 129280x7168, bf16 x")
        if "q6_K_gemm" in want:
            sec["q6_K_gemm"] = gemm_workload(qmv, a.steps, "q6_K prefill GEMM, M=512, 11008x4096 + 4096x11008")
        out["secondary"] = sec
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
