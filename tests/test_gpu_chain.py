"""GPU tests of chain launches (kq_chain_encode / kq_gemv_chain): several
dependent grouped products in one launch, with a grid barrier between
phases. Every logit is checked against the oracle (small shapes) or on
sampled rows (full-size stack layer); chains are bitwise deterministic,
reusable (the barrier count resets itself) and, where the geometry matches,
bitwise equal to the separate grouped launches."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_logits, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_chain(kq, chain, outs):
    for o in outs:
        o.fill_(float("nan"))
    kq.gemv_chain(chain)
    torch.cuda.synchronize()
    assert chain.error_word() == 0, "a chain barrier timed out"
    chain.status()
    return [o.cpu().numpy().copy() for o in outs]


@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_chain_small_ragged_shapes_vs_oracle(kq, layout):
    """Five phases of mixed ragged shapes (partial row groups, one to three
    matrices, two activation widths), m = 16 and m = 3, every logit against
    the oracle; a second run is bitwise identical."""
    lay = kq.LAYOUT_TILED16 if layout == "tiled" else kq.LAYOUT_ROWS
    spec = [(3, 1000, 1024), (1, 300, 2304), (2, 513, 1024), (1, 129, 2304), (2, 700, 2304)]
    xs = {k: synthetic.activations(16, k, 300 + k) for k in (1024, 2304)}
    mats = []
    for pi, (count, n, k) in enumerate(spec):
        mats.append([synthetic.q4k_matrix(n, k, 400 + 10 * pi + j) for j in range(count)])
    for mm in (16, 3):
        log(f"chain small: layout={layout} m={mm}")
        staged = {k: kq.stage_rows(to_dev(x[:mm])) for k, x in xs.items()}
        phases, outs = [], []
        for (count, n, k), ws in zip(spec, mats):
            wd = [to_dev(w) for w in ws]
            if lay == kq.LAYOUT_TILED16:
                wd = [kq.tile_weights(w, n, k) for w in wd]
            lg = [torch.empty((mm, n), dtype=torch.float32, device=DEV) for _ in range(count)]
            phases.append((wd, n, k, staged[k], lg))
            outs.extend(lg)
        chain = kq.chain_encode(phases, mm, layout=lay)
        log(f"chain small: {chain.workgroups} workgroups")
        first = run_chain(kq, chain, outs)
        again = run_chain(kq, chain, outs)
        oi = 0
        for (count, n, k), ws in zip(spec, mats):
            for j in range(count):
                L, A = oracle.gemv_rows(ws[j], k, xs[k][:mm])
                check_logits(first[oi], L, A, what=f"chain phase ({count},{n},{k}) member {j} m={mm}")
                assert np.array_equal(first[oi], again[oi]), "chain not deterministic"
                oi += 1


def test_chain_stack_layer_full_size(kq):
    """One layer of the 52-layer stack as a four-phase chain (q,k,v | o |
    gate,up | down) at full size on tiled weights, as bench.py runs it:
    sampled rows against the oracle at m = 16 and m = 1; row 0 bitwise
    equal between the two; q,k,v, o and down bitwise equal to their
    separate grouped launches when the grid has the same 256 workgroups."""
    mats = synthetic.stack_matrices(1)
    groups = [(0, 1, 2), (3,), (4, 5), (6,)]
    host = {i: synthetic.q4k_matrix(g.n, g.k, g.seed) for i, g in enumerate(mats)}
    wt = {i: kq.tile_weights(to_dev(w), mats[i].n, mats[i].k) for i, w in host.items()}
    ks = sorted({g.k for g in mats})
    xs = {k: synthetic.activations(16, k, synthetic.stack_activation_seed(k)) for k in ks}
    rng = np.random.default_rng(77)
    results = {}
    for mm in (16, 1):
        log(f"chain layer: m={mm}")
        staged = {k: kq.stage_rows(to_dev(xs[k][:mm])) for k in ks}
        phases, outs = [], {}
        for grp in groups:
            g = mats[grp[0]]
            lg = [torch.empty((mm, g.n), dtype=torch.float32, device=DEV) for _ in grp]
            for i, o in zip(grp, lg):
                outs[i] = o
            phases.append(([wt[i] for i in grp], g.n, g.k, staged[g.k], lg))
        chain = kq.chain_encode(phases, mm, layout=kq.LAYOUT_TILED16)
        order = [i for grp in groups for i in grp]
        got = dict(zip(order, run_chain(kq, chain, [outs[i] for i in order])))
        again = dict(zip(order, run_chain(kq, chain, [outs[i] for i in order])))
        results[mm] = got
        for i in order:
            g = mats[i]
            assert np.array_equal(got[i], again[i]), f"matrix {i}: chain not deterministic"
            rows = np.unique(np.concatenate([[0, 1, 127, 128, g.n - 1], rng.integers(0, g.n, 60)]))
            L, A = oracle.gemv_rows(host[i], g.k, xs[g.k][:mm], rows=rows)
            check_logits(got[i][:, rows], L, A, what=f"chain layer matrix {i} ({g.n}x{g.k}) m={mm}")
        if chain.workgroups == 256:
            for grp in ((0, 1, 2), (3,), (6,)):
                g = mats[grp[0]]
                gs = kq.new_group_scratch(g.n, g.k, len(grp), DEV)
                ref = kq.gemv_staged_group([wt[i] for i in grp], g.n, g.k, staged[g.k], mm, gs,
                                           layout=kq.LAYOUT_TILED16)
                torch.cuda.synchronize()
                for i, r in zip(grp, ref):
                    assert np.array_equal(got[i], r.cpu().numpy()), f"matrix {i}: chain != grouped launch"
        else:
            log(f"chain layer: {chain.workgroups} workgroups, grouped-launch bitwise check skipped")
    for i in results[1]:
        assert np.array_equal(results[1][i][0], results[16][i][0]), f"matrix {i}: row 0 depends on m"


def test_chain_many_phases_bitwise_equal_to_single_launches(kq):
    """48 phases (4,096 x 2,048 matrices: 256 units each, so the chain and a
    single launch both use 256 workgroups and cut the work identically):
    every phase bitwise equal to its own launch; the chain runs three times
    in a row (the barrier count must reset itself) with identical results."""
    n, k, n_ph = 4096, 2048, 48
    ws = [synthetic.q4k_matrix(n, k, 900 + i) for i in range(4)]
    wd = [to_dev(w) for w in ws]
    x = synthetic.activations(16, k, 950)
    st = kq.stage_rows(to_dev(x))
    outs = [torch.empty((16, n), dtype=torch.float32, device=DEV) for _ in range(n_ph)]
    phases = [([wd[i % 4]], n, k, st, [outs[i]]) for i in range(n_ph)]
    chain = kq.chain_encode(phases, 16)
    log(f"chain many: {n_ph} phases, {chain.workgroups} workgroups")
    runs = [run_chain(kq, chain, outs) for _ in range(3)]
    scratch = kq.new_scratch(n, k, DEV)
    refs = []
    for i in range(4):
        refs.append(kq.gemv_staged(wd[i], n, k, st, 16, scratch).cpu().numpy())
    rows = np.array([0, 1, 2047, 4095])
    for i in range(4):
        L, A = oracle.gemv_rows(ws[i], k, x, rows=rows)
        check_logits(refs[i][:, rows], L, A, what=f"single launch {i}")
    for r in runs:
        for i in range(n_ph):
            assert np.array_equal(r[i], runs[0][i]), f"phase {i}: runs differ"
            if chain.workgroups == 256:
                assert np.array_equal(r[i], refs[i % 4]), f"phase {i}: chain != single launch"
            else:
                L, A = oracle.gemv_rows(ws[i % 4], k, x, rows=rows)
                check_logits(r[i][:, rows], L, A, what=f"chain many phase {i}")


def test_chain_wait_timeout_sets_error_word_and_reinit_recovers(kq):
    """Failure path, forced from the host: a barrier count preloaded with a
    value no arrival can complete leaves every workgroup waiting for a
    release that never comes; each wait gives up after its bound (1 s of the
    real-time counter), raises the sticky error word and leaves, so the
    launch ends. kq_chain_scratch_init then restores a working state."""
    import time
    n, k = 300, 1024
    w = synthetic.q4k_matrix(n, k, 61)
    x = synthetic.activations(16, k, 62)
    wd = to_dev(w)
    st = kq.stage_rows(to_dev(x))
    outs = [torch.empty((16, n), dtype=torch.float32, device=DEV) for _ in range(2)]
    chain = kq.chain_encode([([wd], n, k, st, [outs[0]]), ([wd], n, k, st, [outs[1]])], 16)
    first = run_chain(kq, chain, outs)
    off = kq.lib.CHAIN_BARRIER_OFFSET
    chain.scratch[off:off + 4].view(torch.int32).fill_(1 << 30)
    torch.cuda.synchronize()
    log("chain timeout: launching with an unreachable barrier count (expect ~1 s)")
    t0 = time.time()
    kq.gemv_chain(chain)
    torch.cuda.synchronize()
    log(f"chain timeout: launch ended after {time.time() - t0:.2f} s")
    assert chain.error_word() == 1
    with pytest.raises(kq.KQError) as e:
        chain.status()
    assert e.value.status == 6  # KQ_ERR_LAUNCH, reported at the C boundary
    chain.init_scratch()
    chain.status()  # cleared: KQ_OK
    again = run_chain(kq, chain, outs)
    for a, b in zip(first, again):
        assert np.array_equal(a, b)
