"""GPU parity of calls with more than 16 activation rows (2 to 4 sixteen-row
slices in one pass over the weights, every format) and of the token-tree
verify (kq_verify_tree_staged) against the oracle: every logit on ragged
shapes, the slices bitwise equal to the same rows of smaller calls of the
same geometry, argmax with flags at the LM-head size for 24 to 64 nodes,
and the tree walk against the oracle's."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_argmax, check_logits, log

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


@pytest.mark.parametrize("fmt,layout", [("q4k", "rows"), ("q4k", "tiled"), ("q5k", "tiled"), ("q6k", "tiled")])
@pytest.mark.parametrize("n,k", [(300, 1024), (1000, 2304), (129, 6656)])
def test_more_rows_every_logit(kq, fmt, layout, n, k):
    w = synthetic.kquant_matrix(fmt, n, k, 700 + n)
    x = synthetic.activations(64, k, 710 + k)
    wd = to_dev(w)
    if layout == "tiled":
        wd = kq.tile_weights(wd, n, k, fmt=fmt)
    lay = kq.FORMATS[fmt][0] if layout == "tiled" else kq.LAYOUT_ROWS
    sc = kq.new_scratch(n, k, DEV)
    L, A = oracle.gemv_rows(w, k, x, fmt=fmt)
    for m in (64, 48, 33, 32, 24, 17):
        log(f"rows: {fmt} {layout} n={n} k={k} m={m}")
        st = kq.stage_rows(to_dev(x[:m]))
        G = kq.gemv_staged(wd, n, k, st, m, sc, layout=lay)
        torch.cuda.synchronize()
        r = check_logits(G.cpu().numpy(), L[:m], A[:m], what=f"{fmt} {layout} n={n} k={k} m={m}")
        log(f"rows: m={m} max |d|/tol = {r:.3g}")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_passes_bitwise_equal_to_smaller_calls(kq, fmt):
    """Calls of 33 to 64 rows make one pass at 3 or 4 slices on the 256-row
    units of a 32-row call, so every 16-row slice equals the same rows of a
    32-row call bit for bit (the same units, the same arithmetic; staging
    scales every row on its own). The 16-row slices of a 32-row call run
    256-row units where a 16-row call runs 128-row units, so they match the
    16-row calls within the oracle's tolerance."""
    n, k = 2000, 6656
    w = synthetic.kquant_matrix(fmt, n, k, 91)
    x = synthetic.activations(64, k, 92)
    wt = kq.tile_weights(to_dev(w), n, k, fmt=fmt)
    lay = kq.FORMATS[fmt][0]
    sc = kq.new_scratch(n, k, DEV)

    def call(rows):
        xs = x[rows]
        return kq.gemv_staged(wt, n, k, kq.stage_rows(to_dev(xs)), len(xs), sc, layout=lay).cpu().numpy()

    g64, g48 = call(slice(0, 64)), call(slice(0, 48))
    g32a, g32b = call(slice(0, 32)), call(slice(32, 64))
    assert np.array_equal(g64[:32], g32a) and np.array_equal(g64[32:], g32b), "64 rows vs two 32-row calls"
    assert np.array_equal(g48[:32], g32a) and np.array_equal(g48[32:], g32b[:16]), "48 rows vs 32-row calls"
    rows = np.array([0, 1, 127, 128, 255, 256, 1999])
    L, A = oracle.gemv_rows(w, k, x[:32], rows=rows, fmt=fmt)
    check_logits(g32a[:, rows], L, A, what=f"{fmt} 32 rows")
    for s in range(2):
        g16 = call(slice(16 * s, 16 * s + 16))
        L16, A16 = oracle.gemv_rows(w, k, x[16 * s:16 * s + 16], rows=rows, fmt=fmt)
        check_logits(g16[:, rows], L16, A16, what=f"{fmt} 16 rows, slice {s}")
        tol = 1e-4 * A16
        assert np.all(np.abs(g32a[16 * s:16 * s + 16][:, rows] - g16[:, rows]) <= 2 * tol), f"slice {s} of 32 rows"
    assert np.array_equal(g64, call(slice(0, 64))), "not deterministic"


@pytest.mark.parametrize("m", [40, 64])
def test_grouped_launch_more_rows(kq, m):
    """Three matrices on one staged block of more than 16 rows in one launch
    (kq_gemv_staged_group): every logit of every member against the oracle."""
    n, k, count = 1000, 2304, 3
    ws = [synthetic.q4k_matrix(n, k, 820 + i) for i in range(count)]
    x = synthetic.activations(m, k, 830)
    wts = [kq.tile_weights(to_dev(w), n, k) for w in ws]
    st = kq.stage_rows(to_dev(x))
    gs = kq.new_group_scratch(n, k, count, DEV)
    got = [g.cpu().numpy() for g in kq.gemv_staged_group(wts, n, k, st, m, gs, layout=kq.LAYOUT_TILED16)]
    for i in range(count):
        L, A = oracle.gemv_rows(ws[i], k, x, fmt="q4k")
        r = check_logits(got[i], L, A, what=f"group m={m} member {i}")
        log(f"group m={m} member {i}: max |d|/tol = {r:.3g}")


def make_tree(rng, m, am, n_vocab, p_follow=0.6):
    """Random tree of m nodes (parent within the 6 previous nodes); a child
    takes its parent's target argmax with probability p_follow (once per
    sibling set), so the walk reaches depth."""
    parent = [-1] + [int(rng.integers(max(0, j - 6), j)) for j in range(1, m)]
    token = [0] * m
    for j in range(1, m):
        used = {token[c] for c in range(1, j) if parent[c] == parent[j]}
        want = int(am[parent[j]])
        if want not in used and rng.random() < p_follow:
            token[j] = want
        else:
            t = int(rng.integers(n_vocab))
            while t in used or t == want:
                t = int(rng.integers(n_vocab))
            token[j] = t
    return parent, token


def test_tree_verify_lm_head(kq):
    """Trees of 24, 32, 33, 40, 48 and 64 nodes on the LM head (6,656 ->
    131,072, Q4_K tiled; one pass over the weights at 2 to 4 slices): argmax of every node row against the oracle (flags), the
    walk equal to the oracle's walk on the GPU's argmax always, and on the
    oracle's argmax when no row is flagged; the path output lists the nodes
    moved through; a chain gives the linear verify's result; the Q6_K head
    at 64 nodes too."""
    h = synthetic.LM_HEAD
    n, k = h["n"], h["k"]
    x = synthetic.activations(64, k, 4242)
    log("tree: oracle over 64 rows of the LM head")
    w = synthetic.q4k_matrix(n, k, h["seed"])
    L, A = oracle.gemv_rows(w, k, x)
    o_am, o_nc = oracle.argmax_flags(L, A)
    log(f"tree: oracle flagged rows {int(np.sum(o_nc > 0))}")
    wt = kq.tile_weights(to_dev(w), n, k)
    sc = kq.new_scratch(n, k, DEV)
    rng = np.random.default_rng(11)
    for m in (24, 32, 33, 40, 48, 64):
        st = kq.stage_rows(to_dev(x[:m]))
        for trial in range(3):
            parent, token = make_tree(rng, m, o_am[:m], n)
            am, acc, path, lg = kq.verify_tree_staged(wt, n, k, st, parent, token, sc, want_logits=(trial == 0),
                                                      layout=kq.LAYOUT_TILED16)
            torch.cuda.synchronize()
            am, acc, path = am.cpu().numpy(), acc.cpu().numpy(), path.cpu().numpy()
            if lg is not None:
                r = check_logits(lg.cpu().numpy(), L[:m], A[:m], what=f"tree logits m={m}")
                log(f"tree: m={m} logits max |d|/tol = {r:.3g}")
            check_argmax(am, L[:m], A[:m], what=f"tree m={m} trial {trial}")
            g_acc, g_nxt, g_path = oracle.tree_accept(parent, token, am)
            assert (int(acc[0]), int(acc[1])) == (g_acc, g_nxt), f"m={m} trial {trial}: walk != oracle walk on GPU argmax"
            assert list(path[:g_acc]) == g_path and np.all(path[g_acc:] == -1)
            if not np.any(o_nc[:m] > 0):
                assert oracle.tree_accept(parent, token, o_am[:m])[:2] == (g_acc, g_nxt)
            log(f"tree: m={m} trial {trial}: accepted {g_acc}, path {g_path}")
        # a chain is the linear verify
        draft = [int(t) for t in o_am[:m - 1]]
        draft[min(m - 2, 20)] = (draft[min(m - 2, 20)] + 1) % n
        am_t, acc_t, _, _ = kq.verify_tree_staged(wt, n, k, st, [-1] + list(range(m - 1)), [0] + draft, sc,
                                                  layout=kq.LAYOUT_TILED16)
        am_l, acc_l, _ = kq.verify_staged(wt, n, k, st, m, draft, sc, layout=kq.LAYOUT_TILED16)
        torch.cuda.synchronize()
        assert np.array_equal(am_t.cpu().numpy(), am_l.cpu().numpy())
        assert np.array_equal(acc_t.cpu().numpy(), acc_l.cpu().numpy())
        assert tuple(acc_l.cpu().numpy()) == oracle.accept(draft, am_l.cpu().numpy())
    del wt
    log("tree: Q6_K head, 64 nodes")
    w6 = synthetic.q6k_matrix(n, k, h["seed"])
    rows = np.arange(n)
    L6, A6 = oracle.gemv_rows(w6, k, x, fmt="q6k")
    o6, n6 = oracle.argmax_flags(L6, A6)
    wt6 = kq.tile_weights(to_dev(w6), n, k, fmt="q6k")
    st = kq.stage_rows(to_dev(x))
    parent, token = make_tree(rng, 64, o6, n)
    am, acc, path, _ = kq.verify_tree_staged(wt6, n, k, st, parent, token, sc, layout=kq.LAYOUT_Q6K_TILED16)
    torch.cuda.synchronize()
    am = am.cpu().numpy()
    check_argmax(am, L6, A6, what="tree q6k m=64")
    assert tuple(acc.cpu().numpy()) == oracle.tree_accept(parent, token, am)[:2]
    del rows


@pytest.mark.parametrize("fmt,m", [("q5k", 48), ("q5k", 64), ("q6k", 40)])
def test_tree_verify_lm_head_q5k_q6k_one_pass(kq, fmt, m):
    """Q5_K and Q6_K LM heads (6,656 -> 131,072) at three and four slices in
    one pass: every logit of every node row within tolerance, the argmax with
    flags, and the walk equal to the oracle's walk on the GPU's argmax."""
    h = synthetic.LM_HEAD
    n, k = h["n"], h["k"]
    x = synthetic.activations(m, k, 4343 + m)
    w = synthetic.kquant_matrix(fmt, n, k, h["seed"] + 7)
    log(f"tree {fmt}: oracle over {m} rows of the LM head")
    L, A = oracle.gemv_rows(w, k, x, fmt=fmt)
    o_am, _ = oracle.argmax_flags(L, A)
    wt = kq.tile_weights(to_dev(w), n, k, fmt=fmt)
    sc = kq.new_scratch(n, k, DEV)
    st = kq.stage_rows(to_dev(x))
    parent, token = make_tree(np.random.default_rng(50 + m), m, o_am, n)
    am, acc, path, lg = kq.verify_tree_staged(wt, n, k, st, parent, token, sc, want_logits=True,
                                              layout=kq.FORMATS[fmt][0])
    torch.cuda.synchronize()
    r = check_logits(lg.cpu().numpy(), L, A, what=f"tree {fmt} logits m={m}")
    am, acc, path = am.cpu().numpy(), acc.cpu().numpy(), path.cpu().numpy()
    check_argmax(am, L, A, what=f"tree {fmt} m={m}")
    g_acc, g_nxt, g_path = oracle.tree_accept(parent, token, am)
    assert (int(acc[0]), int(acc[1])) == (g_acc, g_nxt) and list(path[:g_acc]) == g_path
    log(f"tree {fmt}: m={m} logits max |d|/tol = {r:.3g}, accepted {g_acc}")


@pytest.mark.parametrize("m", [40, 64])
def test_more_than_32_rows_host_staged_and_device_drafts(kq, m):
    """More than 32 rows (one pass at 3 or 4 slices) through the entry
    points that stage the host's x themselves (kq_gemv_rows,
    kq_verify_argmax_accept) and with drafts in device memory
    (kq_verify_staged_dev): every logit within tolerance, the argmax with
    flags, the linear accept equal to the oracle's on the GPU's argmax, with
    a mismatch in the first or the last slices' rows and with every draft
    accepted; the staged and device-draft forms equal the host-staged one
    bit for bit."""
    n, k = 1000, 2304
    w = synthetic.q4k_matrix(n, k, 840 + m)
    x = synthetic.activations(m, k, 850 + m)
    L, A = oracle.gemv_rows(w, k, x)
    w_d, x_d = to_dev(w), to_dev(x)
    G = kq.gemv_rows(w_d, n, k, x_d).cpu().numpy()
    r = check_logits(G, L, A, what=f"gemv_rows m={m}")
    log(f"more rows: gemv_rows m={m} max |d|/tol = {r:.3g}")
    am0, _, _ = kq.verify(w_d, n, k, x_d, [0] * (m - 1))
    am0 = am0.cpu().numpy()
    check_argmax(am0, L, A, what=f"verify m={m}")
    sc = kq.new_scratch(n, k, DEV)
    st = kq.stage_rows(x_d)
    for miss in (m - 3, 20, None):
        draft = [int(t) for t in am0[:m - 1]]
        if miss is not None:
            draft[miss] = (draft[miss] + 1) % n
        am, acc, lg = kq.verify(w_d, n, k, x_d, draft, want_logits=True)
        torch.cuda.synchronize()
        am, acc = am.cpu().numpy(), acc.cpu().numpy()
        assert np.array_equal(am, am0) and np.array_equal(lg.cpu().numpy(), G)
        assert tuple(acc) == oracle.accept(draft, am), f"m={m} miss={miss}"
        am2, acc2, _ = kq.verify_staged(w_d, n, k, st, m, torch.tensor(draft, dtype=torch.int32, device=DEV), sc)
        torch.cuda.synchronize()
        assert np.array_equal(am2.cpu().numpy(), am) and np.array_equal(acc2.cpu().numpy(), acc)
        log(f"more rows: m={m} mismatch at {miss}: accepted {int(acc[0])}, next {int(acc[1])}")


def test_scratch_shared_across_row_counts(kq):
    """One scratch for verify calls of 32, 16, 48, 16, 32 and 48 rows in
    turn. On this shape the one- and two-slice geometries have different
    numbers of row groups, and each call leaves its argmax keys in the
    scratch; with one layout for every call they never land where another
    call expects its zeroed arrival counters. Every call's argmax and accept
    equal the same call on a fresh scratch."""
    n, k = 2000, 2304
    w = synthetic.q4k_matrix(n, k, 870)
    x = synthetic.activations(48, k, 871)
    wt = kq.tile_weights(to_dev(w), n, k)
    shared = kq.new_scratch(n, k, DEV)
    for m in (32, 16, 48, 16, 32, 48):
        st = kq.stage_rows(to_dev(x[:m]))
        fresh = kq.new_scratch(n, k, DEV)
        am_f, acc_f, _ = kq.verify_staged(wt, n, k, st, m, [0] * (m - 1), fresh, layout=kq.LAYOUT_TILED16)
        draft = [int(t) for t in am_f.cpu().numpy()[:m - 1]]
        draft[m - 3] = (draft[m - 3] + 1) % n
        am_f, acc_f, _ = kq.verify_staged(wt, n, k, st, m, draft, fresh, layout=kq.LAYOUT_TILED16)
        am_s, acc_s, _ = kq.verify_staged(wt, n, k, st, m, draft, shared, layout=kq.LAYOUT_TILED16)
        torch.cuda.synchronize()
        assert np.array_equal(am_s.cpu().numpy(), am_f.cpu().numpy()), f"m={m}: argmax on the shared scratch"
        assert np.array_equal(acc_s.cpu().numpy(), acc_f.cpu().numpy()), f"m={m}: accept on the shared scratch"
        assert tuple(acc_s.cpu().numpy()) == (m - 3, int(am_f.cpu().numpy()[m - 3]))
    L, A = oracle.gemv_rows(w, k, x)
    check_argmax(am_s.cpu().numpy(), L, A, what="shared scratch, 48 rows")
