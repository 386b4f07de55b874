#!/usr/bin/env python3
"""Benchmark of the Q4_K batched verify step on one MI355X.

Workload: the synthetic ~16 GB target stack -- 52 layers x (4 x 6,656^2 +
2 x 6,656->17,920 + 1 x 17,920->6,656) Q4_K matrices, then the verify step on
the 6,656 -> 131,072 LM head (argmax of every row + greedy accept of 15 draft
tokens). One step = stage the activation rows (one block per distinct K, the
stack matrices being independent products of a shared input), 364 GEMVs, one
LM-head verify. It runs at M = 16 rows (the headline) and M = 1 (the ratio).

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints one JSON line: verify rows/s at M = 16 (`value`), step times at M = 16
and M = 1, weight GB/s and fraction of the 8 TB/s HBM peak, the dominant
kernel's roofline figure (event-timed per launch) and the CPU oracle timed on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "verify rows/s + weight HBM GB/s (% of peak) at M=1/16; M16÷M1 step-time ratio"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=synthetic.LAYERS)
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a hipGraph")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Stack:
    """Device-resident weights, staged activations, outputs and scratch."""

    def __init__(self, kq, torch, dev, layers):
        self.kq, self.torch, self.dev = kq, torch, dev
        self.mats = synthetic.stack_matrices(layers)
        head = synthetic.LM_HEAD
        self.head = synthetic.Gemv(n=head["n"], k=head["k"], seed=head["seed"])
        t0 = time.time()
        self.w = []
        for i, g in enumerate(self.mats):
            self.w.append(torch.from_numpy(synthetic.q4k_matrix(g.n, g.k, g.seed)).to(dev))
            if i % 50 == 0:
                log(f"bench: generated {i + 1}/{len(self.mats)} matrices ({time.time() - t0:.1f} s)")
        self.w_head = torch.from_numpy(synthetic.q4k_matrix(self.head.n, self.head.k, self.head.seed)).to(dev)
        torch.cuda.synchronize()
        log(f"bench: weights resident ({time.time() - t0:.1f} s)")
        self.ks = sorted({g.k for g in self.mats} | {self.head.k})
        self.x = {k: torch.from_numpy(synthetic.activations(16, k, synthetic.stack_activation_seed(k))).to(dev)
                  for k in self.ks}
        self.staged = {k: kq.lib.alloc_workspace(kq.staged_bytes(k), dev) for k in self.ks}
        shapes = sorted({(g.n, g.k) for g in self.mats})
        self.out = {s: torch.empty((16, s[0]), dtype=torch.float32, device=dev) for s in shapes}
        self.scratch = {s: kq.new_scratch(s[0], s[1], dev) for s in shapes + [(self.head.n, self.head.k)]}
        self.am = torch.empty(16, dtype=torch.int32, device=dev)
        self.acc = torch.empty(2, dtype=torch.int32, device=dev)
        # draft tokens: a seeded random stream of vocabulary ids (acceptance
        # does not change the work a verify step does)
        g = np.random.default_rng(12345)
        self.draft = [int(t) for t in g.integers(0, self.head.n, 15)]
        self.weight_bytes = sum(g.weight_bytes for g in self.mats) + self.head.weight_bytes

    def step(self, m, events=None):
        kq = self.kq
        for k in self.ks:
            kq.stage_rows(self.x[k][:m], staged=self.staged[k])
        for i, g in enumerate(self.mats):
            s = (g.n, g.k)
            if events is not None:
                events[i][0].record()
            kq.gemv_staged(self.w[i], g.n, g.k, self.staged[g.k], m, self.scratch[s], logits=self.out[s][:m])
            if events is not None:
                events[i][1].record()
        h = self.head
        if events is not None:
            events[-1][0].record()
        kq.verify_staged(self.w_head, h.n, h.k, self.staged[h.k], m, self.draft[:m - 1],
                         self.scratch[(h.n, h.k)], out=(self.am[:m], self.acc, None))
        if events is not None:
            events[-1][1].record()

    def algorithmic_bytes(self, m):
        """Per main-kernel launch: weights once + 4*M*K activations + 4*M*N
        logits (not for the LM-head verify, which writes only M+2 ints)."""
        out = [0.5625 * g.n * g.k + 4 * m * g.k + 4 * m * g.n for g in self.mats]
        out.append(0.5625 * self.head.n * self.head.k + 4 * m * self.head.k + 4 * (m + 2))
        return out

    def snapshot(self, m):
        self.torch.cuda.synchronize()
        return (self.am[:m].cpu().numpy().copy(), self.acc.cpu().numpy().copy(),
                {s: o[:m, :64].cpu().numpy().copy() for s, o in self.out.items()})


def same(a, b):
    return (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            and all(np.array_equal(a[2][s], b[2][s]) for s in a[2]))


def timed(torch, fn, steps):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def run_m(stack, torch, m, steps, warmup, use_graph):
    for _ in range(max(1, warmup // 2)):
        stack.step(m)
    eager = stack.snapshot(m)
    if use_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            stack.step(m)  # warm the side stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            stack.step(m)
        for r in range(3):  # every replay must reproduce the eager step
            g.replay()
            snap = stack.snapshot(m)
            if not same(snap, eager):
                raise RuntimeError(f"graph replay {r} differs from the eager step at M={m}")
            stack.step(m)
            torch.cuda.synchronize()
        fn = g.replay
    else:
        def fn():
            stack.step(m)
    for _ in range(warmup):
        fn()
    t = timed(torch, fn, steps)
    if not same(stack.snapshot(m), eager):
        raise RuntimeError(f"timed steps at M={m} changed the results")
    return t


def kernel_roofline(stack, torch, m):
    """Average duration of the main kernel measured with HIP events around
    every launch of one eager step (events on the launch stream)."""
    n = len(stack.mats) + 1
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    stack.step(m, events=ev)
    torch.cuda.synchronize()
    dur = np.array([a.elapsed_time(b) * 1e-3 for a, b in ev])
    byts = np.array(stack.algorithmic_bytes(m))
    avg_s = float(dur.mean())
    avg_b = float(byts.mean())
    ach = avg_b / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "kq_gemv_kernel", "launches": n, "avg_launch_us": round(avg_s * 1e6, 2),
            "avg_algorithmic_bytes": int(avg_b)}


def cpu_baseline(target_s):
    """The oracle (plain C, fp64, OpenMP) on a bounded sample of the step:
    every s-th output row of layer 0's seven matrices and of the LM head, at
    M = 16, on the same bytes the GPU gets. Each matrix's time is scaled by
    its row count to the full matrix; the step is 52 layers plus the head."""
    import oracle
    threads = oracle.num_threads()
    mats = synthetic.stack_matrices(1)
    head = synthetic.LM_HEAD
    shapes = [(g.n, g.k, g.seed) for g in mats] + [(head["n"], head["k"], head["seed"])]
    xs = {k: synthetic.activations(16, k, synthetic.stack_activation_seed(k)) for k in {s[1] for s in shapes}}
    ws = {s: synthetic.q4k_matrix(*s) for s in shapes}

    def run(stride):
        per = []
        for s in shapes:
            n, k, _ = s
            rows = np.arange(0, n, stride)
            t0 = time.perf_counter()
            oracle.gemv_rows(ws[s], k, xs[k], rows=rows)
            per.append((time.perf_counter() - t0) * n / len(rows))
        return synthetic.LAYERS * sum(per[:-1]) + per[-1], sum(len(range(0, s[0], stride)) for s in shapes)

    est, _ = run(256)
    # choose the row stride so that the sample costs about target_s seconds
    stride = int(min(256, max(1, round(256 * (est / 256) / max(target_s, 1e-3) / (synthetic.LAYERS)))))
    t_step, nrows = run(stride)
    return {"value": round(16.0 / t_step, 4), "unit": "verify rows/s", "cores": threads, "kind": "oracle",
            "step_s_extrapolated": round(t_step, 2),
            "sample": f"every {stride}th output row of layer 0's 7 matrices and of the LM head "
                      f"({nrows} rows, M=16, same bytes as the GPU); per-matrix time scaled by row "
                      f"count, step = 52 layers + head"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    import quant_verify_gemv_amd as kq
    kq.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a HIP GPU")
    dev = torch.device("cuda:0")
    stack = Stack(kq, torch, dev, args.layers)
    use_graph = not args.no_graph
    t16 = run_m(stack, torch, 16, args.steps, args.warmup, use_graph)
    log(f"bench: M=16 step {t16 * 1e3:.3f} ms")
    t1 = run_m(stack, torch, 1, args.steps, args.warmup, use_graph)
    log(f"bench: M=1 step {t1 * 1e3:.3f} ms")
    roof = kernel_roofline(stack, torch, 16)
    roof1 = kernel_roofline(stack, torch, 1)
    log(f"bench: roofline M=16 {roof}")
    gbs16 = stack.weight_bytes / t16 / 1e9
    gbs1 = stack.weight_bytes / t1 / 1e9
    cpu = None
    if not args.no_cpu:
        try:
            cpu = cpu_baseline(args.cpu_seconds)
        except Exception as e:  # the baseline must not hide the GPU result
            cpu = {"error": repr(e)}
    rec = {
        "metric": METRIC,
        "value": round(16.0 / t16, 2),
        "unit": "verify rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t16 * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4k-weights/f16x2-mfma/f32-accumulate",
        "data": "synthetic",
        "config": {"workload": f"stack{args.layers}_q4k+lmhead_verify",
                   "matrices": len(stack.mats) + 1,
                   "weight_bytes": stack.weight_bytes,
                   "m": 16, "k_draft": 15, "launch": "hipgraph" if use_graph else "eager"},
        "m16": {"ms_per_step": round(t16 * 1e3, 4), "rows_per_s": round(16 / t16, 2),
                "weight_gb_s": round(gbs16, 1), "hbm_frac": round(gbs16 / HBM_PEAK_GBS, 4)},
        "m1": {"ms_per_step": round(t1 * 1e3, 4), "rows_per_s": round(1 / t1, 2),
               "weight_gb_s": round(gbs1, 1), "hbm_frac": round(gbs1 / HBM_PEAK_GBS, 4),
               "roofline_frac": roof1["frac"]},
        "m16_over_m1": round(t16 / t1, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
