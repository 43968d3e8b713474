#!/usr/bin/env python3
"""Benchmark of the fused dequantize-and-multiply path on one MI355X.

One step = one pass of the decode workload: the three q4_0 GEMVs of a Llama-7B
layer's shapes (4096x4096, 11008x4096, 4096x11008), batch 1, fp32 activations.
Inputs are seeded synthetic planes, uploaded before timing; every step reads a
different copy from a rotating pool of >= 1 GiB so that the 256 MB Infinity Cache
cannot serve repeated reads (the weights come from HBM, as in decode).

Protocol: every workload is set up first; then `--repeats` rounds each measure every
workload once, in the same order (interleaved), and each figure is the median over
the rounds.  Times come from HIP events recorded on the stream the kernels run on,
around replays of HIP graphs that hold the launches; a short spin kernel ahead of the
start event keeps the host's graph submission out of the timed window.

Output: one short progress line per workload while it runs, the full record written to
`--out` (JSON), and as the LAST stdout line a compact JSON record (value = algorithmic
bytes per step / time per step, in GB/s) with `roofline` for the dominant kernel,
`cpu_baseline` (the CPU oracle on a bounded sample, one thread and all threads, plus a
prefill-GEMM leg), the path-label census of every timed launch, and a summary of the
other workloads (q6_K GEMVs, 4-bit codebook MoE, 2-/3-bit additive GEMVs, 8-bit codebook
GEMV, q6_K prefill GEMM).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOPS
POOL_BYTES = 1 << 30           # rotating pool: 4x the 256 MB Infinity Cache
SPIN_CYCLES = 20_000_000       # ~10 ms of GPU spin ahead of each timed replay (a 150-launch graph takes ~1 ms to submit)
LLAMA = [(4096, 4096), (11008, 4096), (4096, 11008)]
EXPERT = [(2048, 7168), (7168, 2048)]
AQ_SHAPES = [(14336, 4096), (4096, 14336)]

METRIC = "quantized GEMV HBM GB/s (% of peak); q6_K prefill GEMM int8 TOPS (% of peak)"
DEFAULT_SECONDARY = "q6_K_gemv,q6_K_decode,q4_0_batch,batch4_other,batch8_other,cb4_moe,aq2x8,aq3x8,cb8,q6_K_gemm"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--repeats", type=int, default=5, help="interleaved rounds; figures are medians")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="per CPU leg")
    ap.add_argument("--only-primary", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--secondary", default=DEFAULT_SECONDARY,
                    help="comma-separated secondary workloads (also: q4_0_q8, aq_lut)")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "bench_full.json"),
                    help="where the full record is written")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, then "
                         "WRITE_SIZE) of `bench.py --only-primary --copy-ref` into the dominant kernel's "
                         "traffic record under profiles/")
    return ap.parse_args()


TRAFFIC_RECORD = os.path.join("profiles", "q4_0_gemv_4096x11008_traffic.json")
TRAFFIC_KERNEL = "gemv_q4_0_kernel<512, 1, 6, 0, true, 1>"  # the 4096x11008 batch-1 launch
TRAFFIC_SOURCES = ["bit_weight_quantized_dequant_amd/csrc/gemv_q4_0.hip",
                   "bit_weight_quantized_dequant_amd/csrc/device_common.h"]


def traffic_summary(fetch_csv, write_csv):
    """HBM bytes per launch of the dominant kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, averaged over its launches), each scaled by what the same counter reads for
    the 256 MiB device copy of --copy-ref (256 MiB read, 256 MiB written)."""
    import csv
    import hashlib

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    kern = [k for k in f if TRAFFIC_KERNEL in k.replace("void ", "").replace("qmv::(anonymous namespace)::", "")]
    copy = [k for k in f if "copy" in k.lower()]
    if len(kern) != 1 or not copy:
        raise SystemExit(f"traffic-summary: kernel {kern!r} / copy {copy!r} not found")
    kern, copy = kern[0], max(copy, key=lambda k: f[k][0])
    ref = 256 << 20
    fetch_scale = ref / 1024 / f[copy][0]
    write_scale = ref / 1024 / w[copy][0]
    traffic = round((f[kern][0] * fetch_scale + w[kern][0] * write_scale) * 1024)
    rec = {
        "kernel": f"{TRAFFIC_KERNEL} at 4096x11008 (q4_0 GEMV, batch 1, fp32 x)",
        "sources_sha256": hashlib.sha256(b"".join(open(os.path.join(ROOT, p), "rb").read()
                                                  for p in TRAFFIC_SOURCES)).hexdigest(),
        "sources": TRAFFIC_SOURCES,
        "launches_sampled": [f[kern][1], w[kern][1]],
        "FETCH_SIZE_KiB_per_launch": round(f[kern][0], 1),
        "WRITE_SIZE_KiB_per_launch": round(w[kern][0], 1),
        "copy_reference": {"bytes_read": ref, "bytes_written": ref, "FETCH_SIZE_KiB": round(f[copy][0], 3),
                           "WRITE_SIZE_KiB": round(w[copy][0], 3)},
        "fetch_scale": round(fetch_scale, 4),
        "write_scale": round(write_scale, 4),
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": 4096 * 11008 // 32 * 18 + 11008 * 4 + 4096 * 4,
        "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py "
                   "--only-primary --copy-ref --steps 8 --warmup 2 --repeats 1 --no-cpu",
    }
    with open(os.path.join(ROOT, TRAFFIC_RECORD), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


T0 = time.perf_counter()


def say(msg: str):
    print(f"[{time.perf_counter() - T0:6.1f} s] {msg}", flush=True)


# ------------------------------------------------------------------ graphs and census

class Census:
    """Path labels of every timed launch: each captured library call records the label the
    library reports for it, and every replay of a graph counts its labels again."""

    def __init__(self):
        self.counts: dict[str, int] = {}
        self.capturing: list | None = None

    def note(self, qmv):
        if self.capturing is not None:
            self.capturing.append(qmv.last_path())

    def add(self, labels, times=1):
        for lab in labels:
            self.counts[lab] = self.counts.get(lab, 0) + times

    def summary(self):
        fb = sum(c for lab, c in self.counts.items() if "fallback" in lab)
        return {"launches": sum(self.counts.values()), "labels": len(self.counts), "fallback": fb}


CENSUS = Census()


class Graph:
    """A HIP graph (torch.cuda.CUDAGraph) replaying fn(0) .. fn(count-1) back to back, with
    the path labels of the launches it holds.  The library enqueues plain kernel launches on
    the current stream, so stream capture records them; replays remove Python's per-launch
    host overhead."""

    def __init__(self, qmv, fn, count):
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(min(count, 3)):
                fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        self.count = count
        CENSUS.capturing = []
        with torch.cuda.graph(self.g):
            for i in range(count):
                fn(i)
        self.labels, CENSUS.capturing = CENSUS.capturing, None
        torch.cuda.synchronize()

    def time(self, warm=True):
        """Milliseconds per item of one replay (HIP events on the replay stream).  A short
        spin kernel runs ahead of the start event, so the host has submitted the whole graph
        before the first timed launch: the events then bracket the launches' execution, not
        the host's submission of them."""
        import torch
        if warm:
            self.g.replay()
            CENSUS.add(self.labels)
            torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN_CYCLES)
        s.record()
        self.g.replay()
        e.record()
        torch.cuda.synchronize()
        CENSUS.add(self.labels)
        return s.elapsed_time(e) / self.count


def med(v):
    return statistics.median(v)


# ------------------------------------------------------------------ inputs

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
    first = dev_planes(synth.gen_weights(fmt, n, k, seed=seed))
    big = {name: torch.empty((copies, *t.shape), dtype=t.dtype, device="cuda") for name, t in first.items()}
    for name, t in first.items():
        big[name][:] = t
    pool = [qmv.QWeights(fmt, n, k, {name: big[name][c] for name in big}) for c in range(copies)]
    pool[0]._keep = big
    return pool


def pool_copies(bytes_per_copy):
    return max(2, -(-POOL_BYTES // bytes_per_copy))


def x_dev(batch, k, xt, seed):
    import torch
    x = synth.gen_x(batch, k, xt, seed=seed)
    if xt == synth.DT_F32:
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()


_POOLS = {}


def shared_pool(qmv, fmt, shapes):
    """One rotating pool per (format, shapes), shared by the workloads (batch sizes) over it."""
    key = (fmt, tuple(shapes))
    if key not in _POOLS:
        per_set = sum(qmv.weight_bytes(fmt, n, k) for n, k in shapes)
        copies = pool_copies(per_set)
        _POOLS[key] = (copies, [make_pool(qmv, fmt, n, k, seed=i, copies=copies) for i, (n, k) in enumerate(shapes)])
    return _POOLS[key]


class ReadCeiling:
    """The stream-read ceiling: the library's read-only kernel over distinct regions of one
    2 GiB buffer (cold, as the GEMV pools), for a given byte count."""

    def __init__(self, qmv):
        import torch
        self.qmv = qmv
        self.buf = torch.zeros(2 << 30, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.graphs = {}

    def graph(self, nbytes, count=60):
        b16 = (nbytes + 15) // 16 * 16
        if b16 not in self.graphs:
            copies = max(2, self.buf.numel() // b16)
            q = self.qmv

            def fn(i):
                q.read_ceiling(self.buf[(i % copies) * b16:(i % copies + 1) * b16], self.sink)
                CENSUS.note(q)
            self.graphs[b16] = Graph(q, fn, count)
        return self.graphs[b16]

    def ms(self, nbytes):
        return self.graph(nbytes).time()

    def graph_uncached(self, nbytes, count=60):
        """A fresh graph (captured under the current forced path) over the same rotation."""
        b16 = (nbytes + 15) // 16 * 16
        copies = max(2, self.buf.numel() // b16)
        q = self.qmv

        def fn(i):
            q.read_ceiling(self.buf[(i % copies) * b16:(i % copies + 1) * b16], self.sink)
            CENSUS.note(q)
        return Graph(q, fn, count)


# ------------------------------------------------------------------ workloads

class GemvWorkload:
    """Batch-`batch` GEMVs over `shapes` (one step = one GEMV per shape), rotating pool;
    per shape, the launch time over the cold pool and the read ceiling for its bytes."""

    def __init__(self, qmv, name, label, fmt, shapes, batch, xt, steps, ceiling, warm_contrast=False, ws=False):
        import torch
        self.qmv, self.name, self.label, self.shapes, self.batch = qmv, name, label, shapes, batch
        copies, mats = shared_pool(qmv, fmt, shapes)
        self.copies = copies
        xb = 4 if xt == synth.DT_F32 else 2
        self.xs = [x_dev(batch, k, xt, seed=i) for i, (n, k) in enumerate(shapes)]
        self.ys = [torch.empty((batch, n), dtype=torch.float32, device="cuda") for n, k in shapes]
        self.algo = [qmv.weight_bytes(fmt, n, k) + xb * batch * k + 4 * batch * n for n, k in shapes]
        self.ceiling = ceiling
        q = qmv
        # ws: qmv_gemv_ws with a workspace per shape (the split-k kernels), else qmv_gemv
        wss = [qmv.gemv_workspace(mats[s][0], batch) for s in range(len(shapes))] if ws else None

        def gemv(s, mat):
            if wss is not None:
                q.gemv_ws(mat, self.xs[s], wss[s], self.ys[s])
            else:
                q.gemv(mat, self.xs[s], self.ys[s])
            CENSUS.note(q)

        def step(i):
            for s in range(len(shapes)):
                gemv(s, mats[s][i % copies])
        self.step_graph = Graph(qmv, step, steps)
        R = max(steps, 40)
        self.shape_graphs, self.warm_graphs = [], []
        for s in range(len(shapes)):
            def one(i, s=s):
                gemv(s, mats[s][i % copies])
            self.shape_graphs.append(Graph(qmv, one, R))
            if warm_contrast:  # the same launches on one copy, which stays in the Infinity Cache
                def warm(i, s=s):
                    gemv(s, mats[s][0])
                self.warm_graphs.append(Graph(qmv, warm, R))
        self.paths = [g.labels[-1] for g in self.shape_graphs]
        self.runs = {"step": [], "shape": [[] for _ in shapes], "warm": [[] for _ in shapes],
                     "ceil": [[] for _ in shapes]}

    def measure(self):
        self.runs["step"].append(self.step_graph.time())
        for s in range(len(self.shapes)):
            self.runs["shape"][s].append(self.shape_graphs[s].time())
            if self.warm_graphs:
                self.runs["warm"][s].append(self.warm_graphs[s].time())
            if self.ceiling is not None:
                self.runs["ceil"][s].append(self.ceiling.ms(self.algo[s]))

    def result(self):
        ms = med(self.runs["step"])
        gbs = sum(self.algo) / ms / 1e6
        shapes = []
        for s, (n, k) in enumerate(self.shapes):
            avg = med(self.runs["shape"][s])
            sh = {"shape": f"{n}x{k}", "bytes": self.algo[s], "avg_launch_ms": round(avg, 5),
                  "runs_ms": [round(v, 5) for v in self.runs["shape"][s]],
                  "GBps": round(self.algo[s] / avg / 1e6, 1), "frac": round(self.algo[s] / avg / 1e6 / HBM_PEAK_GBS, 4),
                  "path": self.paths[s]}
            if self.warm_graphs:
                sh["warm_one_copy_GBps"] = round(self.algo[s] / med(self.runs["warm"][s]) / 1e6, 1)
            if self.runs["ceil"][s]:
                c = med(self.runs["ceil"][s])
                sh["read_ceiling_ms"] = round(c, 5)
                sh["frac_of_read_ceiling"] = round(c / avg, 4)
            shapes.append(sh)
        return {"workload": self.label, "value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "ms_per_step": round(ms, 5), "step_runs_ms": [round(v, 5) for v in self.runs["step"]],
                "bytes_per_step": sum(self.algo), "pool_copies": self.copies, "batch": self.batch,
                "path": self.paths[-1], "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"},
                "shapes": shapes}

    def brief(self):
        r = self.result()
        return [r["value"], r["frac_of_peak"]]


class Q8Workload(GemvWorkload):
    """The GEMV over per-32 int8 activations (q4_0 or q6_K) on the three decode shapes,
    activations quantized beforehand (once per activation vector for every GEMV that reads it)."""

    def __init__(self, qmv, name, label, fmt, batch, steps, ceiling):
        import torch
        self.qmv, self.name, self.label, self.shapes, self.batch = qmv, name, label, LLAMA, batch
        copies, mats = shared_pool(qmv, fmt, LLAMA)
        self.copies = copies
        self.qs = [qmv.quant_act(x_dev(batch, k, synth.DT_F32, seed=i)) for i, (n, k) in enumerate(LLAMA)]
        self.ys = [torch.empty((batch, n), dtype=torch.float32, device="cuda") for n, k in LLAMA]
        self.algo = [qmv.weight_bytes(fmt, n, k) + batch * (k + k // 8) + 4 * batch * n for n, k in LLAMA]
        self.ceiling, self.warm_graphs = ceiling, []
        q = qmv

        def step(i):
            for s in range(len(LLAMA)):
                q.gemv_q8(mats[s][i % copies], self.qs[s][0], self.qs[s][1], self.ys[s])
                CENSUS.note(q)
        self.step_graph = Graph(qmv, step, steps)
        self.shape_graphs = []
        for s in range(len(LLAMA)):
            def one(i, s=s):
                q.gemv_q8(mats[s][i % copies], self.qs[s][0], self.qs[s][1], self.ys[s])
                CENSUS.note(q)
            self.shape_graphs.append(Graph(qmv, one, max(steps, 40)))
        self.paths = [g.labels[-1] for g in self.shape_graphs]
        self.runs = {"step": [], "shape": [[] for _ in LLAMA], "warm": [[] for _ in LLAMA], "ceil": [[] for _ in LLAMA]}


class MoeWorkload:
    """Routed-expert FFN, batch 1: 256 experts of gate/up 2048x7168 and down 7168x2048
    (4-bit codebook, one 16-entry fp16 codebook per 128 weights), top-8 per token.  The
    8.46 GB expert set is resident; its bytes are drawn on the device with a seeded
    generator (throughput does not depend on the values; parity is tested elsewhere)."""

    def __init__(self, qmv, tokens):
        import torch
        E, dm, dff = 256, 7168, 2048
        self.name, self.tokens = "cb4_moe", tokens
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)

        def planes(n, k):
            idx = torch.randint(0, 256, (E, n, k // 2), dtype=torch.uint8, device="cuda", generator=gen)
            cb = torch.randn((E, n, k // 128, 16), device="cuda", generator=gen) * 0.02
            return {"idx": idx, "cb": torch.sort(cb, dim=-1).values.to(torch.float16)}

        self.W = [qmv.QWeights(qmv.CB4, dff, dm, planes(dff, dm)), qmv.QWeights(qmv.CB4, dff, dm, planes(dff, dm)),
                  qmv.QWeights(qmv.CB4, dm, dff, planes(dm, dff))]
        ids = torch.from_numpy(synth.gen_moe_ids(tokens, E, 8, seed=0)).cuda()
        x = torch.from_numpy(synth.gen_x(tokens, dm, synth.DT_BF16, seed=0).view(np.int16).copy()).view(torch.bfloat16).cuda()
        h = torch.empty((8, dff), dtype=torch.float32, device="cuda")
        y = torch.empty((8, dm), dtype=torch.float32, device="cuda")
        self.per_tok = 8 * (qmv.weight_bytes(qmv.CB4, dff, dm) * 2 + qmv.weight_bytes(qmv.CB4, dm, dff)) + 2 * dm + \
            8 * dff * 4 * 2 + 8 * dm * 4
        q, G, U, D = qmv, *self.W

        def step(i):
            q.moe_ffn(G, U, D, E, ids[i % tokens], x[i % tokens], h, y)
            CENSUS.note(q)
        self.g = Graph(qmv, step, tokens)
        self.runs = []

    def measure(self):
        self.runs.append(self.g.time())

    def result(self):
        ms = med(self.runs)
        gbs = self.per_tok / ms / 1e6
        return {"workload": "4-bit codebook MoE FFN, batch 1, 256 experts top-8, gate/up 2048x7168 + down 7168x2048, bf16 x",
                "value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "ms_per_token": round(ms, 5), "runs_ms": [round(v, 5) for v in self.runs],
                "bytes_per_token": self.per_tok, "tokens": self.tokens, "path": self.g.labels[-1],
                "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"}}

    def brief(self):
        r = self.result()
        return [r["value"], r["frac_of_peak"]]


class GemmWorkload:
    """q6_K prefill GEMM, M = 512 tokens, W 11008x4096 and 4096x11008: TOPS = 2 M N K / time.
    The headline is the contraction alone (qmm_gemm_ws on activations the quantizer has put in
    the GEMM's layout) with the weights registered with their pre-expanded planes (the
    default-on registration the method describes).  Beside it: end to end with the quantizer
    (qmm_gemm), the same contraction with the in-kernel expansion (no plane), and with
    row-major int8 activations (qmm_gemm_q8)."""

    def __init__(self, qmv, steps):
        import torch
        self.name, M = "q6_K_gemm", 512
        self.M = M
        self.shapes = [(11008, 4096), (4096, 11008)]
        self.g, self.ops = [], []
        self.keep = []
        q = qmv
        R = max(8, steps // 4)
        for i, (n, k) in enumerate(self.shapes):
            raw = make_pool(qmv, synth.FMT_Q6_K, n, k, seed=i, copies=4)
            exp = make_pool(qmv, synth.FMT_Q6_K, n, k, seed=i, copies=4)
            for W in exp:
                qmv.register_plane(W)
            x = x_dev(M, k, synth.DT_F32, seed=i)
            xq, xs = qmv.quant_act(x)
            y = torch.empty((M, n), dtype=torch.float32, device="cuda")
            ws = torch.empty(qmv.workspace_bytes(raw[0], M), dtype=torch.uint8, device="cuda")
            qmv.gemm(exp[0], x, y, ws)  # leaves the quantized activations in ws
            self.keep += [raw, exp, x, xq, xs, y, ws]

            def plane(j, exp=exp, ws=ws, y=y):
                q.gemm_ws(exp[j % 4], ws, y)
                CENSUS.note(q)

            def e2e(j, exp=exp, x=x, y=y, ws=ws):
                q.gemm(exp[j % 4], x, y, ws)
                CENSUS.note(q)

            def inkernel(j, raw=raw, ws=ws, y=y):
                q.gemm_ws(raw[j % 4], ws, y)
                CENSUS.note(q)

            def rowmajor(j, exp=exp, xq=xq, xs=xs, y=y):
                q.gemm_q8(exp[j % 4], xq, xs, y)
                CENSUS.note(q)
            self.g.append((Graph(qmv, plane, R), Graph(qmv, e2e, R), Graph(qmv, inkernel, R), Graph(qmv, rowmajor, R)))
            self.ops.append(2 * M * n * k)
        self.runs = [[[], [], [], []] for _ in self.shapes]

    def measure(self):
        for s, gs in enumerate(self.g):
            for j, g in enumerate(gs):
                self.runs[s][j].append(g.time())

    def result(self):
        out = {"workload": "q6_K prefill GEMM, M=512, 11008x4096 + 4096x11008", "unit": "TOPS", "shapes": []}
        tot = [0.0, 0.0, 0.0, 0.0]
        for s, (n, k) in enumerate(self.shapes):
            ms = [med(r) for r in self.runs[s]]
            for j in range(4):
                tot[j] += ms[j]
            ops = self.ops[s]
            out["shapes"].append({"shape": f"{n}x{k}", "M": self.M, "ms": round(ms[0], 5), "TOPS": round(ops / ms[0] / 1e9, 1),
                                  "runs_ms": [round(v, 5) for v in self.runs[s][0]],
                                  "path": self.g[s][0].labels[-1], "ms_with_quantizer": round(ms[1], 5),
                                  "ms_in_kernel_expand": round(ms[2], 5),
                                  "TOPS_in_kernel_expand": round(ops / ms[2] / 1e9, 1),
                                  "path_in_kernel_expand": self.g[s][2].labels[-1],
                                  "TOPS_rowmajor_act": round(ops / ms[3] / 1e9, 1)})
        ops = sum(self.ops)
        tops = ops / tot[0] / 1e9
        out.update({"value": round(tops, 1), "frac_of_peak": round(tops / INT8_PEAK_TOPS, 4),
                    "TOPS_with_quantizer": round(ops / tot[1] / 1e9, 1),
                    "TOPS_in_kernel_expand": round(ops / tot[2] / 1e9, 1),
                    "TOPS_rowmajor_act": round(ops / tot[3] / 1e9, 1),
                    "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                                 "frac": round(tops / INT8_PEAK_TOPS, 4)}})
        return out

    def brief(self):
        r = self.result()
        return [r["value"], r["frac_of_peak"], r["TOPS_with_quantizer"], r["TOPS_in_kernel_expand"]]


# ------------------------------------------------------------------ CPU baseline

def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed PMC record, or None
    when the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, TRAFFIC_RECORD)
    try:
        rec = json.load(open(path))
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])).hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    return rec["traffic_bytes_per_launch"] if h == rec["sources_sha256"] else None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds):
    """The oracle as it stands on the host cores: the q4_0 decode step (all rows of the three
    matrices, repeated for about `seconds`) on one thread and on all threads, and the q6_K
    prefill GEMM (quantizer over all 512 x 4096 activations, then a bounded sample of
    (token, row) outputs of the 11008 x 4096 product) on all threads."""
    import oracle
    nth = oracle.max_threads()
    mats, xs, nbytes = [], [], 0
    for i, (n, k) in enumerate(LLAMA):
        mats.append(oracle.Mat(synth.FMT_Q4_0, n, k, synth.gen_weights(synth.FMT_Q4_0, n, k, seed=i)))
        xs.append(synth.gen_x(1, k, seed=i))
        nbytes += (n * k // 32) * 18 + 4 * k + 4 * n

    def leg(threads):
        done, t0 = 0, time.perf_counter()
        while True:
            for m, x in zip(mats, xs):
                oracle.gemv(m, x, oracle.F32, nthreads=threads)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return nbytes * done / el / 1e9, done, el

    v_all, d_all, e_all = leg(nth)
    v_one, d_one, e_one = leg(1)
    # prefill GEMM leg: TOPS over the sampled outputs (2 K int ops each), quantizer included
    n, k, M = 11008, 4096, 512
    gm = oracle.Mat(synth.FMT_Q6_K, n, k, synth.gen_weights(synth.FMT_Q6_K, n, k, seed=0))
    x = synth.gen_x(M, k, seed=0)
    t0 = time.perf_counter()
    xq, xsc = oracle.quant_act(x)
    tq = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    pairs, tg = 0, 0.0
    while tg < seconds:
        mm = rng.integers(0, M, 8192)
        nn = rng.integers(0, n, 8192)
        t0 = time.perf_counter()
        oracle.q6k_gemm_pairs(gm, xq, xsc, mm, nn, nthreads=nth)
        tg += time.perf_counter() - t0
        pairs += len(mm)
    gemm_tops = 2 * k * pairs / tg / 1e12
    return {"value": round(v_all, 3), "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": f"{d_all} full pass(es) of the three q4_0 GEMVs (all rows), fp64 oracle, OpenMP over rows, "
                      f"{e_all:.1f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(v_one, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"{d_one} full pass(es), {e_one:.1f} s"},
            "gemm": {"value": round(gemm_tops, 4), "unit": "TOPS", "cores": nth,
                     "sample": f"{pairs} (token, row) outputs of the 11008x4096 q6_K GEMM at M=512, {tg:.1f} s",
                     "quantizer_ms_512x4096": round(tq * 1e3, 1)}}


# ------------------------------------------------------------------ main

def main():
    a = parse()
    if a.traffic_summary:
        traffic_summary(*a.traffic_summary)
        return
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
        del src, dst

    t_start = time.perf_counter()
    ceiling = None if a.only_primary else ReadCeiling(qmv)
    # the primary workload: warm-up steps, then `steps` timed steps per round
    prim = GemvWorkload(qmv, "q4_0_step", "q4_0 GEMV batch 1, Llama-7B decode shapes 4096x4096 + 11008x4096 + "
                        "4096x11008, fp32 x, rotating HBM pool", synth.FMT_Q4_0, LLAMA, 1, synth.DT_F32,
                        a.steps, ceiling, warm_contrast=True)
    copies, mats = shared_pool(qmv, synth.FMT_Q4_0, LLAMA)
    xw = prim.xs

    def warm_step(i):
        for s in range(len(LLAMA)):
            qmv.gemv(mats[s][(i + 1000) % copies], xw[s], prim.ys[s])
            CENSUS.note(qmv)
    Graph(qmv, warm_step, max(1, a.warmup)).time(warm=False)
    say(f"bench: primary set up ({copies} pool copies)")

    work = [prim]
    want = set() if a.only_primary else set(a.secondary.split(","))
    steps2 = 50

    def add(w):
        work.append(w)
        say(f"bench: set up {w.name}")

    if "q6_K_gemv" in want:
        add(GemvWorkload(qmv, "q6_K_gemv", "q6_K GEMV batch 1, 256x1024, fp32 x", synth.FMT_Q6_K, [(256, 1024)], 1,
                         synth.DT_F32, 200, ceiling))
    if "q6_K_decode" in want:
        for b in (1, 4, 8) if "batch8_other" in want else (1, 4):
            add(GemvWorkload(qmv, f"q6_K_gemv_b{b}", f"q6_K GEMV batch {b}, Llama-7B decode shapes, fp32 x",
                             synth.FMT_Q6_K, LLAMA, b, synth.DT_F32, steps2, ceiling))
    if "q4_0_batch" in want:
        for b in (2, 4, 8):
            add(GemvWorkload(qmv, f"q4_0_gemv_b{b}", f"q4_0 GEMV batch {b}, Llama-7B decode shapes, fp32 x",
                             synth.FMT_Q4_0, LLAMA, b, synth.DT_F32, steps2, ceiling))
    if "q4_0_q8" in want:
        for b in (1, 4):
            add(Q8Workload(qmv, f"q4_0_q8_gemv_b{b}", f"q4_0 GEMV over per-32 int8 activations, batch {b}, "
                           "Llama-7B decode shapes", synth.FMT_Q4_0, b, steps2, ceiling))
    if "cb4_moe" in want:
        add(MoeWorkload(qmv, 64))
    for fmt, nm, label in ((synth.FMT_AQ2X8, "aq2x8", "2-bit additive"), (synth.FMT_AQ3X8, "aq3x8", "3-bit additive")):
        if nm in want:
            bs = (1, 4, 8) if (nm == "aq2x8" and "batch8_other" in want) else (1, 4)
            for b in bs:
                add(GemvWorkload(qmv, f"{nm}_gemv_b{b}", f"{label} GEMV batch {b}, 14336x4096 + 4096x14336, bf16 x",
                                 fmt, AQ_SHAPES, b, synth.DT_BF16, steps2, ceiling))
        if "aq_lut" in want:
            add(GemvWorkload(qmv, f"{nm}_lut_gemv_b1", f"{label} GEMV batch 1 through per-slice lookup tables "
                             "(qmv_gemv_ws, split k), 14336x4096 + 4096x14336, bf16 x",
                             fmt, AQ_SHAPES, 1, synth.DT_BF16, steps2, ceiling, ws=True))
    for fmt, nm, label in ((synth.FMT_CB4, "cb4", "4-bit codebook"), (synth.FMT_CB8, "cb8", "8-bit codebook")):
        for b in [b for b, tag in ((4, "batch4_other"), (8, "batch8_other")) if tag in want]:
            add(GemvWorkload(qmv, f"{nm}_gemv_b{b}", f"{label} GEMV batch {b}, 2048x7168 + 7168x2048, bf16 x",
                             fmt, EXPERT, b, synth.DT_BF16, steps2, ceiling))
    if "cb8" in want:
        add(GemvWorkload(qmv, "cb8_gemv", "8-bit codebook GEMV batch 1, shared expert gate/up 2048x7168 + down "
                         "7168x2048 and output head 129280x7168, bf16 x", synth.FMT_CB8,
                         [(2048, 7168), (2048, 7168), (7168, 2048), (129280, 7168)], 1, synth.DT_BF16, 20, ceiling))
    if "q6_K_gemm" in want:
        add(GemmWorkload(qmv, a.steps))

    # interleaved rounds: every workload once per round, in the same order
    for r in range(max(1, a.repeats)):
        for w in work:
            w.measure()
        say(f"bench: round {r + 1}/{a.repeats} done, primary {sum(prim.algo) / prim.runs['step'][-1] / 1e6:.1f} GB/s")
    gpu_s = time.perf_counter() - t_start

    pr = prim.result()
    dom = max(pr["shapes"], key=lambda s: s["avg_launch_ms"])
    full = {
        "metric": METRIC,
        "value": pr["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "repeats": a.repeats,
        "ms_per_step": pr["ms_per_step"],
        "step_runs_ms": pr["step_runs_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": pr["workload"], "batch": 1, "pool_copies": pr["pool_copies"],
                   "bytes_per_step": pr["bytes_per_step"]},
        "frac_of_peak": pr["frac_of_peak"],
        "roofline": {"bound": "hbm", "kernel": f"q4_0 GEMV {dom['shape']} ({dom['path']})",
                     "achieved": dom["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom["frac"],
                     "traffic": recorded_traffic() if dom["shape"] == "4096x11008" else None,
                     "read_ceiling_frac": dom.get("frac_of_read_ceiling")},
        "shapes": pr["shapes"],
        "secondary": {w.name: w.result() for w in work[1:]},
        "census": {"counts": CENSUS.counts, **CENSUS.summary()},
        "gpu_seconds": round(gpu_s, 1),
    }
    if ceiling is not None:
        big = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")

        def rd(i):
            qmv.read_ceiling(big, sink)
            CENSUS.note(qmv)
        ms = med([Graph(qmv, rd, 5).time() for _ in range(3)])
        full["read_ceiling_4GiB_GBps"] = round(big.numel() / ms / 1e6, 1)
        del big
        # the ceiling's own check: persistent grids with 2 or 4 loads in flight per lane
        # against one load per thread, at the primary shapes' sizes
        sweep = {}
        for n, k in LLAMA:
            nb = qmv.weight_bytes(synth.FMT_Q4_0, n, k)
            row = {}
            for variant in ("", "read-ceiling.persistent-u2", "read-ceiling.persistent-u4"):
                os.environ["QMV_FORCE_PATH"] = variant
                try:
                    g = ReadCeiling.graph_uncached(ceiling, nb)
                    row[g.labels[-1]] = round(nb / med([g.time() for _ in range(3)]) / 1e6, 1)
                finally:
                    os.environ.pop("QMV_FORCE_PATH", None)
            sweep[f"{n}x{k}"] = row
        full["read_ceiling_variants_GBps"] = sweep
    if not a.no_cpu:
        say("bench: timing the CPU oracle")
        full["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        json.dump(full, f, indent=1)

    # the compact record, last line of stdout
    line = {k: full[k] for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                                 "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                                 "frac_of_peak", "roofline")}
    line["repeats"] = a.repeats
    line["shapes_GBps"] = {s["shape"]: s["GBps"] for s in pr["shapes"]}
    if "cpu_baseline" in full:
        cb = full["cpu_baseline"]
        line["cpu_baseline"] = {"value": cb["value"], "unit": cb["unit"], "cores": cb["cores"], "kind": cb["kind"],
                                "sample": "q4_0 step, all rows, fp64 oracle", "cpu_model": cb["cpu_model"],
                                "one_thread_GBps": cb["one_thread"]["value"], "gemm_TOPS": cb["gemm"]["value"]}
    line["census"] = CENSUS.summary()
    line["secondary"] = {"fields": "GB/s, frac of 8 TB/s (GEMM: TOPS, frac of 5 POPS, TOPS with the quantizer, "
                                   "TOPS without planes)", **{w.name: w.brief() for w in work[1:]}}
    line["full_record"] = os.path.relpath(os.path.abspath(a.out), ROOT)
    print(json.dumps(line, separators=(",", ":")))


if __name__ == "__main__":
    main()
