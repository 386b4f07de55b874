#!/usr/bin/env python3
"""Benchmark of the Q4_K batched verify step on one MI355X.

Workload: the synthetic ~16 GB target stack -- 52 layers x (4 x 6,656^2 +
2 x 6,656->17,920 + 1 x 17,920->6,656) Q4_K matrices, then the verify step on
the 6,656 -> 131,072 LM head (argmax of every row + greedy accept of 15 draft
tokens). One step = stage the activation rows (one block per distinct K, the
stack matrices being independent products of a shared input), 364 GEMVs in
208 dependent phases (one chain launch by default), one LM-head verify. It
runs at M = 16 rows (the headline) and M = 1 (the ratio).

The stack follows a transformer layer's data dependencies: the three
projections that read the same hidden state (q, k, v) form one phase, the
output projection the next, gate and up the next, down the last -- four
phases per layer, 208 for the stack. By default the whole stack is one chain
launch (kq_gemv_chain: a grid barrier between consecutive phases, so each
phase reads its activations only after the previous phase's outputs are
complete); --launch grouped issues one launch per phase instead. Then the
LM-head verify.

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
# plain Q4_K products of the 128-row geometry (the square and fc shapes) run
# on the chain kernel's one-phase mode
ONE_PHASE = "kq_chain_kernel (one-phase launch)"
METRIC = "verify rows/s + weight HBM GB/s (% of peak) at M=1/16; M16÷M1 step-time ratio"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=synthetic.LAYERS)
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a hipGraph")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extras", action="store_true",
                   help="only the timed steps (no per-step spread, draft-block or read-probe timing): "
                        "the dispatch sequence the counter passes expect")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--m", choices=("both", "16", "1"), default="both", help="row counts to time")
    p.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                   help="weight layout: the tiled copy (default) or llama.cpp's row-major blocks")
    p.add_argument("--launch", choices=("chain", "grouped"), default="chain",
                   help="stack as one chain launch (default) or one launch per phase")
    p.add_argument("--copy-probe", action="store_true",
                   help="first run plain 1 GiB device copies (counter calibration under rocprofv3 --pmc)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Stack:
    """Device-resident weights, staged activations, outputs and scratch."""

    def __init__(self, kq, torch, dev, layers, layout, launch="chain", on_matrix=None, keep_rows=False):
        """`on_matrix(i, gemv, w_host)` is called with each matrix's host
        bytes before they are uploaded (a parity check computes its oracle
        rows there, so the 16 GB of host bytes need not be kept)."""
        self.kq, self.torch, self.dev = kq, torch, dev
        self.layout = layout
        self.launch = launch
        # keep_rows: also keep the llama.cpp row-layout copy of every matrix
        # resident (the row-layout figures)
        self.keep_rows = keep_rows and layout == kq.LAYOUT_TILED16
        self.w_rows = []
        self.mats = synthetic.stack_matrices(layers)
        head = synthetic.LM_HEAD
        self.head = synthetic.Gemv(n=head["n"], k=head["k"], seed=head["seed"])
        t0 = time.time()
        self.w = []
        for i, g in enumerate(self.mats):
            w_host = synthetic.q4k_matrix(g.n, g.k, g.seed)
            if on_matrix is not None:
                on_matrix(i, g, w_host)
            self.w.append(self.resident(w_host, g.n, g.k))
            del w_host
            if i % 50 == 0:
                log(f"bench: generated {i + 1}/{len(self.mats)} matrices ({time.time() - t0:.1f} s)")
        w_host = synthetic.q4k_matrix(self.head.n, self.head.k, self.head.seed)
        if on_matrix is not None:
            on_matrix(len(self.mats), self.head, w_host)
        self.w_head = self.resident(w_host, self.head.n, self.head.k)
        del w_host
        torch.cuda.synchronize()
        log(f"bench: weights resident ({time.time() - t0:.1f} s)")
        self.ks = sorted({g.k for g in self.mats} | {self.head.k})
        self.x = {k: torch.from_numpy(synthetic.activations(16, k, synthetic.stack_activation_seed(k))).to(dev)
                  for k in self.ks}
        self.staged = {k: kq.lib.alloc_workspace(kq.staged_bytes(k), dev) for k in self.ks}
        # launch groups: matrix indices within a layer that share one launch
        self.groups = []
        for layer in range(layers):
            base = 7 * layer
            for idx in ((0, 1, 2), (3,), (4, 5), (6,)):
                self.groups.append(tuple(base + i for i in idx))
        keys = sorted({(self.mats[g[0]].n, self.mats[g[0]].k, len(g)) for g in self.groups})
        # one output buffer per matrix (every logit of the step stays
        # available for the parity check: 230 MB at M = 16)
        self.out = [torch.empty((16, g.n), dtype=torch.float32, device=dev) for g in self.mats]
        self.scratch = {kk: kq.new_group_scratch(kk[0], kk[1], kk[2], dev) for kk in keys}
        self.chains = {}
        self.head_scratch = kq.new_scratch(self.head.n, self.head.k, dev)
        self.am = torch.empty(16, dtype=torch.int32, device=dev)
        self.acc = torch.empty(2, dtype=torch.int32, device=dev)
        # draft tokens: a seeded random stream of vocabulary ids (acceptance
        # does not change the work a verify step does)
        g = np.random.default_rng(12345)
        self.draft = [int(t) for t in g.integers(0, self.head.n, 15)]
        self.weight_bytes = sum(g.weight_bytes for g in self.mats) + self.head.weight_bytes

    def resident(self, w_host, n, k):
        """Device copy of a Q4_K matrix in the benchmark's weight layout (the
        tiled copy is made once, outside the timed region, as an engine would
        when it loads weights)."""
        w = self.torch.from_numpy(w_host).to(self.dev)
        if self.layout == self.kq.LAYOUT_TILED16:
            t = self.kq.tile_weights(w, n, k)
            if self.keep_rows:
                self.w_rows.append(w)
            del w
            return t
        return w

    @property
    def launches(self):
        """Launches of the main kernel per step."""
        return (1 if self.launch == "chain" else len(self.groups)) + 1

    def chain(self, m):
        """The stack as one chain (encoded once per m)."""
        if m not in self.chains:
            phases = []
            for grp in self.groups:
                g = self.mats[grp[0]]
                phases.append(([self.w[j] for j in grp], g.n, g.k, self.staged[g.k],
                               [self.out[j][:m] for j in grp]))
            self.chains[m] = self.kq.chain_encode(phases, m, layout=self.layout)
        return self.chains[m]

    def step(self, m):
        kq = self.kq
        for k in self.ks:
            kq.stage_rows(self.x[k][:m], staged=self.staged[k])
        if self.launch == "chain":
            kq.gemv_chain(self.chain(m))
        else:
            for grp in self.groups:
                g = self.mats[grp[0]]
                key = (g.n, g.k, len(grp))
                kq.gemv_staged_group([self.w[j] for j in grp], g.n, g.k, self.staged[g.k], m, self.scratch[key],
                                     logits=[self.out[j][:m] for j in grp], layout=self.layout)
        h = self.head
        kq.verify_staged(self.w_head, h.n, h.k, self.staged[h.k], m, self.draft[:m - 1],
                         self.head_scratch, out=(self.am[:m], self.acc, None), layout=self.layout)

    def algorithmic_bytes(self, m):
        """Per main-kernel launch: every matrix's weights once, the M
        activation rows once (4*M*K) and the M fp32 logit rows of every
        matrix (4*M*N each); the LM-head verify writes M + 2 ints instead."""
        out = []
        for grp in self.groups:
            g = self.mats[grp[0]]
            out.append(len(grp) * (0.5625 * g.n * g.k + 4 * m * g.n) + 4 * m * g.k)
        if self.launch == "chain":
            out = [sum(out)]
        out.append(0.5625 * self.head.n * self.head.k + 4 * m * self.head.k + 4 * (m + 2))
        return out

    def snapshot(self, m):
        self.torch.cuda.synchronize()
        return (self.am[:m].cpu().numpy().copy(), self.acc.cpu().numpy().copy(),
                {j: o[:m, :64].cpu().numpy().copy() for j, o in enumerate(self.out)})


def same(a, b):
    return (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            and all(np.array_equal(a[2][s], b[2][s]) for s in a[2]))


def timed(torch, fn, steps):
    """Wall time per step (host clock, synchronized on both sides) and HIP
    event time per step (events on the stream the kernels run on)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, e0.elapsed_time(e1) * 1e-3 / steps


def run_m(stack, torch, m, steps, warmup, use_graph, extras=True):
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
    wall, ev = timed(torch, fn, steps)
    if not same(stack.snapshot(m), eager):
        raise RuntimeError(f"timed steps at M={m} changed the results")
    if stack.launch == "chain":
        stack.chain(m).status()  # raises KQError when a chain wait gave up
    if not extras:
        return wall, ev, None
    # spread over steps: each of `steps` further steps between its own events
    # (outside the timed region above)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    spread = {"median_ms": round(float(np.median(per)), 4), "p95_ms": round(float(np.percentile(per, 95)), 4),
              "cv": round(float(per.std() / per.mean()), 4) if len(per) > 1 else 0.0}
    return wall, ev, spread


def graph_time(torch, fn, calls, reps=5):
    """Microseconds per call: `calls` back-to-back calls fn(0..calls-1)
    captured in one HIP graph, averaged over `reps` replays timed with HIP
    events on the replay stream (so the host's per-call cost of the Python
    binding is not in the figure)."""
    for i in range(3):
        fn(i)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * calls)


def positive_control(stack, torch):
    """The all-accept instrument check, reported apart from the results: the
    LM-head verify at M = 16 with the draft set to the target's own argmax of
    rows 0..14 must accept all 15 and emit row 15's argmax."""
    kq, h = stack.kq, stack.head
    sth = stack.staged[h.k]
    kq.stage_rows(stack.x[h.k][:16], staged=sth)
    am, _, _ = kq.verify_staged(stack.w_head, h.n, h.k, sth, 16, stack.draft[:15], stack.head_scratch,
                                layout=stack.layout)
    own = [int(v) for v in am.cpu().numpy()]
    am2, acc2, _ = kq.verify_staged(stack.w_head, h.n, h.k, sth, 16, own[:15], stack.head_scratch,
                                    layout=stack.layout)
    got = [int(v) for v in acc2.cpu().numpy()]
    ok = got == [15, own[15]] and [int(v) for v in am2.cpu().numpy()] == own
    if not ok:
        raise RuntimeError(f"positive control: accept {got}, expected [15, {own[15]}]")
    return {"draft": "the target's own argmax of rows 0-14", "accepted": got[0], "next_token": got[1], "ok": ok}


def draft_block_timing(stack, torch, calls=50):
    """The draft block's proposals (argmax of rows 1..15 of a 16-row block
    against the LM head, no accept), timed on the resident LM-head weights
    and checked bitwise against the verify step's argmax of the same rows."""
    kq = stack.kq
    h = stack.head
    st = stack.staged[h.k]
    kq.stage_rows(stack.x[h.k][:16], staged=st)
    props = torch.empty(15, dtype=torch.int32, device=stack.dev)
    head = torch.empty(1, dtype=torch.int32, device=stack.dev)

    def call():
        kq.draft_block_argmax_staged(stack.w_head, h.n, h.k, st, 15, stack.head_scratch, want_head=True,
                                     out=(props, head), layout=stack.layout)
    for _ in range(5):
        call()
    kq.verify_staged(stack.w_head, h.n, h.k, st, 16, stack.draft[:15], stack.head_scratch,
                     out=(stack.am, stack.acc, None), layout=stack.layout)
    torch.cuda.synchronize()
    same_rows = bool(torch.equal(props, stack.am[1:16]) and torch.equal(head, stack.am[:1]))
    if not same_rows:
        raise RuntimeError("draft block proposals differ from the verify step's argmax of the same rows")
    us = graph_time(torch, lambda i: call(), calls)
    gbs = h.weight_bytes / (us * 1e-6) / 1e9
    return {"verify_length": 15, "us_per_call": round(us, 2), "weight_gb_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "calls": calls, "launch": "hipgraph, back-to-back",
            "matches_verify_argmax": same_rows}


def config_timings(stack, torch, calls=50):
    """The other configurations of the benchmark definition, each timed on
    its own (back-to-back launches replayed from a HIP graph, tiled
    weights as in the step): the square 6,656 x 6,656 product at every M of
    its sweep, rotating over 16 copies (399 MB, more than the 256 MB MALL),
    and at M = 1 and 16 on one resident copy (the hot-cache figure, labelled);
    the DFlash fc projection 33,280 -> 6,656 at M = 16 over 4 copies
    (498 MB); and the LM-head verify at M = 16 on the resident head (491 MB).
    Each result: microseconds per call, verify rows/s, weight GB/s and its
    fraction of the 8 TB/s peak."""
    kq = stack.kq
    dev = stack.dev
    out = {}

    def rate(nbytes, m, us, alg=None, kernel="kq_gemv_kernel"):
        """nbytes: weight bytes per call; alg: algorithmic bytes per call
        (weights + activations + outputs) for the roofline point."""
        gbs = nbytes / (us * 1e-6) / 1e9
        r = {"us_per_call": round(us, 2), "rows_per_s": round(m / (us * 1e-6), 1),
             "weight_gb_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if alg is not None:
            r["roofline"] = roofline_entry(kernel, alg, us)
        return r

    def time_calls(fn):
        return graph_time(torch, fn, calls)

    def copies(cfg, count):
        n, k = cfg["n"], cfg["k"]
        return [kq.tile_weights(torch.from_numpy(synthetic.q4k_matrix(n, k, cfg["seed"] + 100 * c)).to(dev), n, k)
                for c in range(count)]

    sq = synthetic.SQUARE
    n, k = sq["n"], sq["k"]
    ws = copies(sq, 16)
    wbytes = n * synthetic.q4k_bytes_per_row(k)
    x = torch.from_numpy(synthetic.activations(16, k, sq["seed"])).to(dev)
    scratch = kq.new_scratch(n, k, dev)
    logits = torch.empty((16, n), dtype=torch.float32, device=dev)
    res = {}
    for m in sq["ms"]:
        st = kq.stage_rows(x[:m])
        us = time_calls(lambda i: kq.gemv_staged(ws[i % 16], n, k, st, m, scratch, logits=logits[:m],
                                                   layout=kq.LAYOUT_TILED16))
        res[f"m{m}"] = rate(wbytes, m, us, wbytes + 4 * m * (n + k), kernel=ONE_PHASE)
    res["m16_over_m1"] = round(res["m16"]["us_per_call"] / res["m1"]["us_per_call"], 4)
    out["square_6656x6656"] = res
    # the same product on one copy every call: its 25 MB stay in the 256 MB
    # MALL, so this is a cache figure (labelled, no HBM roofline point)
    hot = {}
    for m in (1, 16):
        st = kq.stage_rows(x[:m])
        us = time_calls(lambda i: kq.gemv_staged(ws[0], n, k, st, m, scratch, logits=logits[:m],
                                                   layout=kq.LAYOUT_TILED16))
        hot[f"m{m}"] = {key: v for key, v in rate(wbytes, m, us).items() if key != "hbm_frac"}
    hot["note"] = "one resident copy (25 MB, within the 256 MB MALL): a cache figure, not an HBM rate"
    out["square_6656x6656_hot_cache"] = hot
    del ws
    fc = synthetic.FC
    n, k = fc["n"], fc["k"]
    ws = copies(fc, 4)
    xf = torch.from_numpy(synthetic.fc_activations(16, fc["seed"])).to(dev)
    st = kq.stage_rows(xf)
    scratch = kq.new_scratch(n, k, dev)
    logits = torch.empty((16, n), dtype=torch.float32, device=dev)
    us = time_calls(lambda i: kq.gemv_staged(ws[i % 4], n, k, st, 16, scratch, logits=logits,
                                               layout=kq.LAYOUT_TILED16))
    out["fc_33280_to_6656_m16"] = rate(n * synthetic.q4k_bytes_per_row(k), 16, us,
                                       n * synthetic.q4k_bytes_per_row(k) + 4 * 16 * (n + k), kernel=ONE_PHASE)
    del ws
    h = stack.head
    sth = stack.staged[h.k]
    kq.stage_rows(stack.x[h.k][:16], staged=sth)
    us = time_calls(lambda i: kq.verify_staged(stack.w_head, h.n, h.k, sth, 16, stack.draft[:15], stack.head_scratch,
                                                 out=(stack.am, stack.acc, None), layout=stack.layout))
    out["lm_head_verify_m16"] = rate(h.weight_bytes, 16, us, h.weight_bytes + 4 * 16 * h.k + 4 * 18,
                                     kernel="kq_gemv_kernel (LM-head verify)")
    out["stochastic_lm_head_m16"] = stochastic_timing(stack, torch, time_calls)
    out.update(kquant_timings(stack, torch, time_calls))
    tree = out["tree_verify_lm_head"]
    tree["m64_over_lm_head_m16"] = round(tree["m64"]["us_per_call"] / out["lm_head_verify_m16"]["us_per_call"], 4)
    out["launch"] = "hipgraph, back-to-back"
    torch.cuda.synchronize()
    return out


def kquant_timings(stack, torch, time_calls):
    """The Q5_K and Q6_K paths on the benchmark's shapes: the square
    6,656 x 6,656 product at M = 1 and 16 over 16 rotating copies of each
    format, and the LM-head verify (6,656 -> 131,072, M = 16, k = 15) with
    Q6_K weights (the output layer's usual k-quant) and a 64-node token tree
    on it. Weight bytes per call are the format's own (176 or 210 per 256
    weights). Then the token-tree verify of 24, 32, 48 and 64 nodes on the
    resident Q4_K LM head (rows/s counts the tree's nodes)."""
    kq = stack.kq
    dev = stack.dev
    out = {}

    def rate(nbytes, m, us, alg=None):
        gbs = nbytes / (us * 1e-6) / 1e9
        r = {"us_per_call": round(us, 2), "rows_per_s": round(m / (us * 1e-6), 1),
             "weight_gb_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if alg is not None:
            r["roofline"] = roofline_entry("kq_gemv_kernel", alg, us)
        return r

    sq = synthetic.SQUARE
    n, k = sq["n"], sq["k"]
    x = torch.from_numpy(synthetic.activations(16, k, sq["seed"])).to(dev)
    scratch = kq.new_scratch(n, k, dev)
    logits = torch.empty((16, n), dtype=torch.float32, device=dev)
    for fmt in ("q5k", "q6k"):
        layout, bb = kq.FORMATS[fmt]
        ws = [kq.tile_weights(torch.from_numpy(synthetic.kquant_matrix(fmt, n, k, sq["seed"] + 100 * c)).to(dev),
                              n, k, fmt=fmt) for c in range(16)]
        res = {}
        for m in (1, 16):
            st = kq.stage_rows(x[:m])
            us = time_calls(lambda i: kq.gemv_staged(ws[i % 16], n, k, st, m, scratch, logits=logits[:m],
                                                       layout=layout))
            res[f"m{m}"] = rate(n * (k // 256) * bb, m, us, n * (k // 256) * bb + 4 * m * (n + k))
        out[f"square_6656x6656_{fmt}"] = res
        del ws
    h = stack.head
    w6 = kq.tile_weights(torch.from_numpy(synthetic.q6k_matrix(h.n, h.k, h.seed)).to(dev), h.n, h.k, fmt="q6k")
    sth = stack.staged[h.k]
    kq.stage_rows(stack.x[h.k][:16], staged=sth)
    us = time_calls(lambda i: kq.verify_staged(w6, h.n, h.k, sth, 16, stack.draft[:15], stack.head_scratch,
                                                 out=(stack.am, stack.acc, None), layout=kq.LAYOUT_Q6K_TILED16))
    out["lm_head_verify_m16_q6k"] = rate(h.n * (h.k // 256) * 210, 16, us,
                                         h.n * (h.k // 256) * 210 + 4 * 16 * h.k + 4 * 18)
    # a 64-node token tree on the same Q6_K head, all nodes in one pass
    g6 = np.random.default_rng(78)
    x6 = torch.from_numpy(synthetic.activations(64, h.k, 4242)).to(dev)
    parent6 = [-1] + [int(g6.integers(max(0, j - 6), j)) for j in range(1, 64)]
    token6 = [0] + [int(t) for t in g6.integers(0, h.n, 63)]
    st6 = kq.stage_rows(x6)
    am6 = torch.empty(64, dtype=torch.int32, device=dev)
    acc6 = torch.empty(2, dtype=torch.int32, device=dev)
    path6 = torch.empty(64, dtype=torch.int32, device=dev)
    us = time_calls(lambda i: kq.verify_tree_staged(w6, h.n, h.k, st6, parent6, token6, stack.head_scratch,
                                                      out=(am6, acc6, path6, None), layout=kq.LAYOUT_Q6K_TILED16))
    t6 = rate(h.n * (h.k // 256) * 210, 64, us, h.n * (h.k // 256) * 210 + 4 * 64 * h.k + 4 * (2 * 64 + 2))
    t6["m64_over_lm_head_m16_q6k"] = round(us / out["lm_head_verify_m16_q6k"]["us_per_call"], 4)
    out["tree_verify_lm_head_q6k_m64"] = t6
    del w6
    # token-tree verify on the resident Q4_K head: a tree of m nodes (parent
    # within the previous 6 nodes, seeded tokens), all nodes in one pass
    g = np.random.default_rng(77)
    x64 = torch.from_numpy(synthetic.activations(64, h.k, 4242)).to(dev)
    tree = {}
    for m in (24, 32, 48, 64):
        parent = [-1] + [int(g.integers(max(0, j - 6), j)) for j in range(1, m)]
        token = [0] + [int(t) for t in g.integers(0, h.n, m - 1)]
        st = kq.stage_rows(x64[:m])
        am = torch.empty(m, dtype=torch.int32, device=dev)
        acc = torch.empty(2, dtype=torch.int32, device=dev)
        path = torch.empty(m, dtype=torch.int32, device=dev)
        us = time_calls(lambda i: kq.verify_tree_staged(stack.w_head, h.n, h.k, st, parent, token, stack.head_scratch,
                                                          out=(am, acc, path, None), layout=stack.layout))
        tree[f"m{m}"] = rate(h.weight_bytes, m, us, h.weight_bytes + 4 * m * h.k + 4 * (2 * m + 2))
    out["tree_verify_lm_head"] = tree
    torch.cuda.synchronize()
    return out


def stochastic_timing(stack, torch, time_calls, temperature=300.0, decisions=20):
    """The stochastic verify at the LM-head size (16 rows x 131,072): the
    verify launch with logits out, the target probability rows
    (kq_softmax_rows: two launches, 8 algorithmic bytes per element, one
    fp32 read and one write), and the library's host decision
    (kq_speculative_decide) on rows copied to host memory, with the copy
    timed on its own; then the same decisions in two steps (kq_gather_rows
    of p_i[d_i] on the device, those k values and the one row the decision
    walks copied to the host, kq_speculative_first_reject and
    kq_speculative_resample), checked equal. Draft rows are the softmax of
    perturbed logits."""
    kq = stack.kq
    h = stack.head
    n, m = h.n, 16
    sth = stack.staged[h.k]
    lg = torch.empty((m, n), dtype=torch.float32, device=stack.dev)
    probs = torch.empty_like(lg)
    ws = torch.empty(max(256, kq.softmax_workspace_bytes(m, n)), dtype=torch.uint8, device=stack.dev)
    us_verify = time_calls(lambda i: kq.verify_staged(stack.w_head, n, h.k, sth, m, stack.draft[:15],
                                                      stack.head_scratch, out=(stack.am, stack.acc, lg),
                                                      layout=stack.layout))
    us_soft = time_calls(lambda i: kq.softmax_rows(lg, temperature, 0.0, probs=probs, workspace=ws))

    def both(i):
        kq.verify_staged(stack.w_head, n, h.k, sth, m, stack.draft[:15], stack.head_scratch,
                         out=(stack.am, stack.acc, lg), layout=stack.layout)
        kq.softmax_rows(lg, temperature, 0.0, probs=probs, workspace=ws)
    us_both = time_calls(both)
    gen = torch.Generator(device=stack.dev).manual_seed(5)
    noisy = lg[:m - 1] + 60.0 * torch.randn((m - 1, n), generator=gen, device=stack.dev)
    q = kq.softmax_rows(noisy.contiguous(), temperature).cpu().numpy()
    torch.cuda.synchronize()
    host = torch.empty((m, n), dtype=torch.float32, pin_memory=True)
    t0 = time.perf_counter()
    for _ in range(decisions):
        host.copy_(probs)
    us_copy = (time.perf_counter() - t0) * 1e6 / decisions
    p = host.numpy()
    orders = np.argsort(-p, axis=1, kind="stable").astype(np.int32)
    rng = np.random.default_rng(9)
    drafts = [[int(np.searchsorted(np.cumsum(q[i], dtype=np.float64), rng.random() * q[i].sum()))
               for i in range(m - 1)] for _ in range(decisions)]
    drafts = [[min(t, n - 1) for t in d] for d in drafts]
    us_ = rng.random((decisions, m)).astype(np.float32)
    t0 = time.perf_counter()
    decided = [kq.speculative_decide(drafts[j], q, p, orders, us_[j]) for j in range(decisions)]
    us_decide = (time.perf_counter() - t0) * 1e6 / decisions
    accepted = [a for a, _ in decided]
    # the same decisions in two steps: p_i[d_i] gathered on the device, k
    # values and then the one row the decision walks copied to the host
    kd = m - 1
    drafts_d = [torch.tensor(d, dtype=torch.int32, device=stack.dev) for d in drafts]
    q_at = [q[np.arange(kd), d] for d in drafts]
    pat_h = torch.empty(kd, dtype=torch.float32, pin_memory=True)
    row_h = torch.empty(n, dtype=torch.float32, pin_memory=True)
    torch.cuda.synchronize()
    t_copy = t_host = 0.0
    for j in range(decisions):
        t0 = time.perf_counter()
        pat_h.copy_(kq.gather_rows(probs[:kd], drafts_d[j]))
        pos = kq.speculative_first_reject(pat_h.numpy(), q_at[j], us_[j][:kd])
        row_h.copy_(probs[pos])
        t1 = time.perf_counter()
        tok = (kq.speculative_resample(row_h.numpy(), q[pos], orders[pos], us_[j][pos + 1]) if pos < kd
               else kq.speculative_resample(row_h.numpy(), None, orders[kd], us_[j][kd]))
        t_host += time.perf_counter() - t1
        t_copy += t1 - t0
        if (pos, tok) != decided[j]:
            raise RuntimeError("the two-step decision differs from the full-row decision")
    soft_bytes = 8 * m * n
    return {"temperature": temperature,
            "verify_logits_us": round(us_verify, 2),
            "softmax_rows_us": round(us_soft, 2),
            "softmax_gb_s": round(soft_bytes / (us_soft * 1e-6) / 1e9, 1),
            "softmax_algorithmic_bytes": soft_bytes,
            "verify_plus_rows_us": round(us_both, 2),
            "rows_to_host_us": round(us_copy, 1),
            "host_decide_us": round(us_decide, 1),
            "gather_and_one_row_to_host_us": round(t_copy * 1e6 / decisions, 1),
            "host_resample_us": round(t_host * 1e6 / decisions, 1),
            "mean_accepted": round(float(np.mean(accepted)), 2)}


def rows_layout_timing(stack, torch, steps):
    """The step streamed from llama.cpp's row-major blocks, next to the
    tiled headline: (a) the same chain with KQ_LAYOUT_ROWS (its outputs are
    checked bitwise against the tiled chain's: the layouts give identical
    results), and (b) the step as the boundary's two all-in-one entry
    points make it, kq_gemv_rows per stack matrix (each stages its own
    activations) and kq_verify_argmax_accept on the LM head, 365 calls in
    one HIP graph. M = 16 and M = 1; milliseconds per step and weight GB/s."""
    kq = stack.kq
    out = {}
    if not stack.w_rows:
        return None
    w_head_rows = stack.w_rows[-1]
    ws = {}
    for g in stack.mats + [stack.head]:
        key = (g.n, g.k)
        if key not in ws:
            ws[key] = kq.lib.alloc_workspace(kq.workspace_bytes(g.n, g.k, 16), stack.dev)
    for m in (16, 1):
        for k in stack.ks:
            kq.stage_rows(stack.x[k][:m], staged=stack.staged[k])
        phases = []
        for grp in stack.groups:
            g = stack.mats[grp[0]]
            phases.append(([stack.w_rows[j] for j in grp], g.n, g.k, stack.staged[g.k],
                           [stack.out[j][:m] for j in grp]))
        chain = kq.chain_encode(phases, m, layout=kq.LAYOUT_ROWS)
        ref = None
        if stack.launch == "chain":
            kq.gemv_chain(stack.chain(m))
            torch.cuda.synchronize()
            ref = [o[:m, :64].cpu().numpy().copy() for o in stack.out]
        us_chain = event_us(torch, lambda: kq.gemv_chain(chain), max(3, steps // 4))
        chain.status()
        if ref is not None:
            for j, o in enumerate(stack.out):
                if not np.array_equal(o[:m, :64].cpu().numpy(), ref[j]):
                    raise RuntimeError(f"row-layout chain differs from the tiled chain (matrix {j}, M={m})")
        h = stack.head
        am = torch.empty(m, dtype=torch.int32, device=stack.dev)
        acc = torch.empty(2, dtype=torch.int32, device=stack.dev)

        def boundary_step(_i):
            for j, g in enumerate(stack.mats):
                kq.gemv_rows(stack.w_rows[j], g.n, g.k, stack.x[g.k][:m], logits=stack.out[j][:m],
                             workspace=ws[(g.n, g.k)])
            kq.verify(w_head_rows, h.n, h.k, stack.x[h.k][:m], stack.draft[:m - 1], workspace=ws[(h.n, h.k)],
                      out=(am, acc, None))
        us_b = graph_time(torch, boundary_step, 1, reps=max(3, steps // 4))
        # the head verify is not in the chain launch: add its row-layout time
        us_head = graph_time(torch, lambda i: kq.verify_staged(w_head_rows, h.n, h.k, stack.staged[h.k], m,
                                                                stack.draft[:m - 1], stack.head_scratch,
                                                                out=(am, acc, None), layout=kq.LAYOUT_ROWS), 20)
        step_chain = us_chain + us_head
        out[f"m{m}"] = {
            "chain_rows_ms_per_step": round(step_chain * 1e-3, 4),
            "chain_rows_weight_gb_s": round(stack.weight_bytes / (step_chain * 1e-6) / 1e9, 1),
            "chain_rows_hbm_frac": round(stack.weight_bytes / (step_chain * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "boundary_calls_ms_per_step": round(us_b * 1e-3, 4),
            "boundary_calls_weight_gb_s": round(stack.weight_bytes / (us_b * 1e-6) / 1e9, 1),
            "boundary_calls_hbm_frac": round(stack.weight_bytes / (us_b * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del chain
    out["note"] = ("chain_rows: the headline's chain launch plus the LM-head verify, weights in llama.cpp rows; "
                   "boundary_calls: kq_gemv_rows x 364 + kq_verify_argmax_accept (each call stages its own "
                   "activations), one HIP graph")
    torch.cuda.synchronize()
    return out


def read_ceiling(stack, torch, calls=20):
    """Pure-read rate of this device on the resident LM-head weights (the
    library's read probe: every byte loaded once): the achievable ceiling
    the weight stream is compared with, reported next to the roofline."""
    kq = stack.kq
    buf = stack.w_head
    sink = kq.stream_probe(buf)
    for _ in range(3):
        kq.stream_probe(buf, sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        kq.stream_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / calls
    nbytes = buf.numel() * buf.element_size()
    gbs = nbytes / s / 1e9
    return {"gb_s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "buffer": "LM-head weights as streamed", "calls": calls}


def source_digest():
    """sha256 over the kernel sources and the launch-geometry code: a stored
    traffic figure is only valid for the code it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in ("kq_kernels.hip", "kq_internal.h", "kq_api.cpp"):
        with open(os.path.join(ROOT, "quant_verify_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload, m, layout_name, launch):
    """HBM bytes of one launch (`launch`: "chain" or "lm_head") from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE scaled by the
    copy-kernel calibration), or None when there is none for this workload
    and M or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"kq_chain_kernel.{workload}.traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != source_digest() or vals.get("weight_layout") != layout_name:
        return None
    v = vals.get(f"traffic_bytes_{launch}_m{m}")
    return float(v) if v else None


def roofline_entry(kernel, algorithmic_bytes, us, launches=1, traffic=None):
    """One kernel's roofline point: algorithmic bytes per launch / its own
    average launch duration (HIP events on the stream it runs on)."""
    ach = algorithmic_bytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "avg_launch_us": round(us, 3), "launches": launches, "algorithmic_bytes": int(algorithmic_bytes)}


def event_us(torch, fn, reps):
    """Microseconds per call of fn(), eager, between two HIP events on the
    current stream (for launches long enough that the host's per-call cost
    hides behind the GPU: the chain launch)."""
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def kernel_rooflines(stack, torch, m, reps, workload, layout_name):
    """Every kernel of the step timed on its own, at M = m: the stack (one
    chain launch, or the 208 grouped launches), the LM-head verify, and the
    activation staging (one launch per distinct K). Each gets its own
    roofline point; their sum is compared with the step time."""
    kq = stack.kq
    for k in stack.ks:
        kq.stage_rows(stack.x[k][:m], staged=stack.staged[k])
    out = {}
    if stack.launch == "chain":
        ch = stack.chain(m)
        us = event_us(torch, lambda: kq.gemv_chain(ch), reps)
        ch.status()
        out["stack_chain"] = roofline_entry("kq_chain_kernel (208 phases)", stack.algorithmic_bytes(m)[0], us,
                                            1, stored_traffic(workload, m, layout_name, "chain"))
    else:
        def grouped():
            for grp in stack.groups:
                g = stack.mats[grp[0]]
                key = (g.n, g.k, len(grp))
                kq.gemv_staged_group([stack.w[j] for j in grp], g.n, g.k, stack.staged[g.k], m, stack.scratch[key],
                                     logits=[stack.out[j][:m] for j in grp], layout=stack.layout)
        us = graph_time(torch, lambda i: grouped(), 1, reps=reps) / len(stack.groups)
        out["stack_grouped"] = roofline_entry("kq_gemv_kernel (grouped, per launch)",
                                              float(np.mean(stack.algorithmic_bytes(m)[:-1])), us, len(stack.groups))
    h = stack.head
    us = graph_time(torch, lambda i: kq.verify_staged(stack.w_head, h.n, h.k, stack.staged[h.k], m,
                                                      stack.draft[:m - 1], stack.head_scratch,
                                                      out=(stack.am[:m], stack.acc, None), layout=stack.layout), 50)
    out["lm_head_verify"] = roofline_entry("kq_gemv_kernel (LM-head verify)", stack.algorithmic_bytes(m)[-1], us, 1,
                                           stored_traffic(workload, m, layout_name, "lm_head"))
    x_bytes = sum(4 * m * k + kq.staged_bytes(k) for k in stack.ks)
    us = graph_time(torch, lambda i: [kq.stage_rows(stack.x[k][:m], staged=stack.staged[k]) for k in stack.ks], 20)
    out["stage"] = roofline_entry("kq_stage_kernel (all distinct K)", x_bytes, us, len(stack.ks))
    out["sum_us"] = round(sum(v["avg_launch_us"] * v["launches"] for v in out.values() if isinstance(v, dict)), 2)
    return out


def copy_probe(torch, dev, nbytes=1 << 30):
    """Plain device copies of known size, for calibrating the FETCH_SIZE and
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copy probe {nbytes} bytes x 3")


def launch_geometry_record(stack) -> dict:
    """The geometry the timed launches actually used: the chain's persistent
    workgroups, and the LM-head verify's waves, tiles per wave, workgroups
    and units (one row group by one 256-column block)."""
    kq, h = stack.kq, stack.head
    waves, tpw, wgs, units = kq.launch_geometry(h.n, h.k)
    rec = {"lm_head_verify": {"waves": waves, "tiles_per_wave": tpw, "rows_per_group": 16 * waves * tpw,
                              "workgroups": wgs, "units": units}}
    if stack.launch == "chain":
        rec["stack_chain"] = {"workgroups": stack.chain(16).workgroups, "rows_per_group": 128,
                              "phases": len(stack.groups)}
    return rec


def device_info(torch) -> dict:
    """The GPU and software the numbers were measured on."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": torch.cuda.get_device_name(0), "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count, "memory_gib": round(pr.total_memory / 2 ** 30, 1),
            "hip": torch.version.hip, "torch": torch.__version__}


def host_cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s, check=None):
    """The oracle (plain C, fp64, OpenMP) on a bounded sample of the step, at
    M = 16, on the same bytes the GPU gets: the LM head in full and whole
    stack layers, as many as fit in about target_s seconds. The step time is
    52 x the mean layer time + the head time (exact when all layers ran).
    check(i, L, A) is called, outside the timed calls, with the oracle's
    logits and tolerance mass of every matrix it ran (i = stack index, or
    None for the LM head)."""
    import oracle
    threads = oracle.num_threads()
    head = synthetic.LM_HEAD
    xs = {k: synthetic.activations(16, k, synthetic.stack_activation_seed(k))
          for k in (synthetic.HIDDEN, synthetic.FFN)}

    def timed_gemv(i, n, k, seed):
        w = synthetic.q4k_matrix(n, k, seed)
        t0 = time.perf_counter()
        L, A = oracle.gemv_rows(w, k, xs[k])
        t = time.perf_counter() - t0
        if check is not None:
            check(i, L, A)
        return t

    t_head = timed_gemv(None, head["n"], head["k"], head["seed"])
    mats = synthetic.stack_matrices(synthetic.LAYERS)
    layer_times = []
    spent = t_head
    for layer in range(synthetic.LAYERS):
        t = sum(timed_gemv(7 * layer + j, g.n, g.k, g.seed) for j, g in enumerate(mats[7 * layer:7 * layer + 7]))
        layer_times.append(t)
        spent += t
        if spent + float(np.mean(layer_times)) > target_s:
            break
    t_step = synthetic.LAYERS * float(np.mean(layer_times)) + t_head
    # one core: a 6,656 x 6,656 matrix at 1 thread and at all threads; the
    # step scales by that ratio
    g0 = mats[3]
    w0 = synthetic.q4k_matrix(g0.n, g0.k, g0.seed)
    t_all = time.perf_counter()
    oracle.gemv_rows(w0, g0.k, xs[g0.k], threads=threads)
    t_all = time.perf_counter() - t_all
    t_one = time.perf_counter()
    oracle.gemv_rows(w0, g0.k, xs[g0.k], threads=1)
    t_one = time.perf_counter() - t_one
    t_step1 = t_step * t_one / t_all
    wbytes = sum(g.weight_bytes for g in mats) + head["n"] * synthetic.q4k_bytes_per_row(head["k"])
    # the other configurations: the oracle's median of 3 runs each (generation
    # outside the timed calls)
    per_config = {}
    t_configs = 0.0
    for name, cfg, m, x in (("tiny", synthetic.TINY, 4, None), ("square_m16", synthetic.SQUARE, 16, None),
                            ("fc_m16", synthetic.FC, 16, synthetic.fc_activations(16, synthetic.FC["seed"])),
                            ("lm_head_m16", head, 16, None)):
        w = synthetic.q4k_matrix(cfg["n"], cfg["k"], cfg["seed"])
        x = synthetic.activations(m, cfg["k"], cfg["seed"]) if x is None else x
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.gemv_rows(w, cfg["k"], x, threads=threads)
            times.append(time.perf_counter() - t0)
        t = float(np.median(times))
        t_configs += sum(times)
        per_config[name] = {"ms": round(t * 1e3, 3), "rows_per_s": round(m / t, 2),
                            "weight_gb_s": round(w.nbytes / t / 1e9, 3)}
    return {"value": round(16.0 / t_step, 4), "unit": "verify rows/s", "cores": threads, "kind": "oracle",
            "cpu_model": host_cpu_model(), "weight_gb_s": round(wbytes / t_step / 1e9, 3),
            "step_s_extrapolated": round(t_step, 3), "sample_s": round(spent + t_all + t_one + t_configs, 2),
            "sample": f"LM head in full + {len(layer_times)} of {synthetic.LAYERS} stack layers in full "
                      f"(M=16, same bytes as the GPU); step = {synthetic.LAYERS} x mean layer time + head",
            "configs": per_config,
            "single_core": {"value": round(16.0 / t_step1, 5), "weight_gb_s": round(wbytes / t_step1 / 1e9, 4),
                            "step_s_extrapolated": round(t_step1, 2),
                            "sample": f"one {g0.n} x {g0.k} matrix at 1 thread ({t_one:.2f} s) and at {threads} "
                                      f"({t_all:.3f} s); the step scaled by that ratio"}}


class StepCheck:
    """Parity of the timed step at M = 16 against the oracle outputs the CPU
    baseline computes anyway: every logit of every stack matrix it ran
    within 1e-4 * sum_k |w_k x_k|, and the LM head's argmax (ties within the
    tolerance may resolve to any candidate) and accept decision."""

    def __init__(self, stack, outs, am, acc):
        self.stack, self.outs, self.am, self.acc = stack, outs, am, acc
        self.matrices = 0
        self.logits = 0
        self.worst = 0.0
        self.head = None

    def __call__(self, i, L, A):
        import oracle
        if i is None:
            o_am, o_nc = oracle.argmax_flags(L, A)
            flagged = []
            for r in range(L.shape[0]):
                ok = int(self.am[r]) == int(o_am[r])
                if o_nc[r]:
                    flagged.append(r)
                    ok = ok or int(self.am[r]) in set(int(c) for c in oracle.candidates(L[r], A[r], int(o_am[r])))
                if not ok:
                    raise RuntimeError(f"parity: LM-head row {r} argmax {self.am[r]} != oracle {o_am[r]}")
            draft = self.stack.draft[:15]
            acc_g = oracle.accept(draft, [int(v) for v in self.am])
            if tuple(int(v) for v in self.acc) != acc_g:
                raise RuntimeError("parity: the accept decision does not follow the GPU's argmaxes")
            acc_o = oracle.accept(draft, [int(v) for v in o_am])
            exact = not any(o_nc[:acc_o[0] + 1])
            if exact and acc_g != acc_o:
                raise RuntimeError(f"parity: accept {acc_g} != oracle {acc_o}")
            self.head = {"argmax_rows": int(L.shape[0]), "flagged_rows": flagged, "accept": list(acc_g),
                         "accept_equals_oracle": acc_g == acc_o}
            return
        G = self.outs[i].astype(np.float64)
        err = np.abs(G - L)
        tol = 1e-4 * A
        if not np.all(err <= tol):
            bad = np.argwhere(err > tol)[0]
            raise RuntimeError(f"parity: stack matrix {i} logit {tuple(bad)} off by {err[tuple(bad)]!r} "
                               f"> tolerance {tol[tuple(bad)]!r}")
        self.worst = max(self.worst, float(np.max(err / np.maximum(tol, 1e-300))))
        self.matrices += 1
        self.logits += int(G.size)

    def result(self):
        return {"against": "oracle (cpu_baseline's own outputs, M = 16)", "stack_matrices": self.matrices,
                "logits": self.logits, "max_err_over_tol": float(f"{self.worst:.3g}"), "lm_head": self.head}


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
    if args.copy_probe:
        copy_probe(torch, dev)
    layout = kq.LAYOUT_TILED16 if args.layout == "tiled" else kq.LAYOUT_ROWS
    stack = Stack(kq, torch, dev, args.layers, layout, args.launch, keep_rows=not args.no_extras)
    use_graph = not args.no_graph
    workload = f"stack{args.layers}_q4k+lmhead_verify"
    layout_name = "tiled16" if layout == kq.LAYOUT_TILED16 else "rows"
    res = {}
    snap16 = None
    for m in ((16, 1) if args.m == "both" else (int(args.m),)):
        wall, ev, spread = run_m(stack, torch, m, args.steps, args.warmup, use_graph, not args.no_extras)
        if m == 16 and not args.no_cpu:
            # every output of the timed steps, for the parity check against
            # the oracle outputs of the CPU baseline (outside the timed region)
            torch.cuda.synchronize()
            snap16 = ([o.cpu().numpy() for o in stack.out], stack.am.cpu().numpy().copy(),
                      stack.acc.cpu().numpy().copy())
        gbs = stack.weight_bytes / wall / 1e9
        res[m] = {"ms_per_step": round(wall * 1e3, 4), "rows_per_s": round(m / wall, 2),
                  "weight_gb_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                  "event_ms_per_step": round(ev * 1e3, 4), "step_spread": spread}
        if not args.no_extras:
            kr = kernel_rooflines(stack, torch, m, max(5, args.steps // 2), workload, layout_name)
            res[m]["kernels"] = kr
            res[m]["roofline"] = kr["stack_chain" if args.launch == "chain" else "stack_grouped"]
            log(f"bench: M={m} step {wall * 1e3:.3f} ms (events {ev * 1e3:.3f} ms), {gbs:.1f} GB/s; kernels "
                + ", ".join(f"{k} {v['avg_launch_us']} us ({v['frac']})" for k, v in kr.items() if isinstance(v, dict)))
        else:
            log(f"bench: M={m} step {wall * 1e3:.3f} ms (events {ev * 1e3:.3f} ms), {gbs:.1f} GB/s")
    draft = ceiling = cfgs = rows_fig = control = None
    if not args.no_extras:
        control = positive_control(stack, torch)
        log("bench: positive control " + json.dumps(control))
        draft = draft_block_timing(stack, torch)
        ceiling = read_ceiling(stack, torch)
        rows_fig = rows_layout_timing(stack, torch, args.steps)
        log("bench: row layout " + json.dumps(rows_fig))
        cfgs = config_timings(stack, torch)
        log("bench: configs " + json.dumps(cfgs))
        log(f"bench: read ceiling {ceiling['gb_s']} GB/s ({ceiling['frac']:.3f} of peak)")
        log(f"bench: draft block proposals {draft['us_per_call']} us/call, {draft['weight_gb_s']} GB/s")
    cpu = parity = None
    if not args.no_cpu:
        check = StepCheck(stack, *snap16) if snap16 is not None else None
        try:
            cpu = cpu_baseline(args.cpu_seconds, check)
        except RuntimeError as e:
            if str(e).startswith("parity:"):
                raise  # a wrong result produces no bench line
            cpu = {"error": repr(e)}
        except Exception as e:  # the baseline must not hide the GPU result
            cpu = {"error": repr(e)}
        if check is not None and "error" not in cpu:
            parity = check.result()
            log(f"bench: parity vs oracle: {json.dumps(parity)}")
    head_m = 16 if 16 in res else min(res)
    top = res[head_m]
    rec = {
        "metric": METRIC,
        "value": top["rows_per_s"],
        "unit": "verify rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": top["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4k-weights/f16x2-mfma/f32-accumulate",
        "data": "synthetic",
        "config": {"workload": workload,
                   "matrices": len(stack.mats) + 1, "launches_per_step": stack.launches + len(stack.ks),
                   "weight_bytes": stack.weight_bytes,
                   "m": head_m, "k_draft": head_m - 1, "launch": "hipgraph" if use_graph else "eager",
                   "stack_launch": args.launch,
                   "weight_layout": "tiled16" if layout == kq.LAYOUT_TILED16 else "llama.cpp rows"},
        "m16": res.get(16),
        "m1": res.get(1),
        "m16_over_m1": round(res[16]["ms_per_step"] / res[1]["ms_per_step"], 4) if len(res) == 2 else None,
        "roofline": top.get("roofline"),
        "read_ceiling": ceiling,
        "positive_control": control,
        "draft_block_argmax": draft,
        "configs": cfgs,
        "rows_layout": rows_fig,
        "cpu_baseline": cpu,
        "device": device_info(torch),
        "geometry": launch_geometry_record(stack),
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
