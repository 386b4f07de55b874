"""Seeded random shapes against the oracle.

Row counts are drawn log-uniform from 1 to 150,000, depths from one block up
to a bounded matrix size, activation rows from 1 to 64 and the format from
Q4_K, Q5_K and Q6_K. That mixes launches with fewer units than workgroups,
row groups split over one to many workgroups, ragged last tiles, every row
geometry and one to four activation slices per pass, in
combinations no hand-picked shape list covers. Each case checks every logit
of the staged product, the row-major calls bitwise against the tiled one,
the verify's argmax (with flags) and accept, and for more than 16 rows a
random token tree's walk. Chains of several phases of mixed random shapes
are checked the same way, phase by phase."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_accept, check_argmax, check_logits, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_WEIGHTS = 24_000_000  # weights per matrix: keeps the oracle at a second or so


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def draw_shape(rng, max_m=64, n_max=150_000):
    n = max(1, int(np.exp(rng.uniform(0.0, np.log(n_max)))))
    kb = int(rng.integers(1, max(1, min(48, MAX_WEIGHTS // (256 * n))) + 1))
    if max_m <= 16 or rng.random() < 0.75:
        m = int(rng.integers(1, min(16, max_m) + 1))
    else:
        m = int(rng.integers(17, max_m + 1))
    return n, 256 * kb, m


def random_tree(rng, m, am, n_vocab, p_follow=0.6):
    """m nodes, each node's parent among the 6 before it; a child takes its
    parent's target argmax with probability p_follow, else a uniform token
    (siblings may repeat a token; the walk then takes the lowest index)."""
    parent = [-1] + [int(rng.integers(max(0, j - 6), j)) for j in range(1, m)]
    token = [0] * m
    for j in range(1, m):
        token[j] = int(am[parent[j]]) if rng.random() < p_follow else int(rng.integers(n_vocab))
    return parent, token


@pytest.mark.parametrize("seed", range(64))
def test_random_shape(kq, seed):
    rng = np.random.default_rng(50_000 + seed)
    n, k, m = draw_shape(rng)
    fmt = ("q4k", "q4k", "q5k", "q6k")[int(rng.integers(4))]
    geom = kq.launch_geometry(n, k)
    log(f"random shape seed={seed}: {fmt} n={n} k={k} m={m} geometry {geom}")
    w = synthetic.kquant_matrix(fmt, n, k, 51_000 + seed)
    x = synthetic.activations(m, k, 52_000 + seed)
    L, A = oracle.gemv_rows(w, k, x, fmt=fmt)
    o_am, o_nc = oracle.argmax_flags(L, A)
    lay = kq.FORMATS[fmt][0]
    w_d, x_d = to_dev(w), to_dev(x)
    wt = kq.tile_weights(w_d, n, k, fmt=fmt)
    st = kq.stage_rows(x_d)
    sc = kq.new_scratch(n, k, DEV)

    G = kq.gemv_staged(wt, n, k, st, m, sc, layout=lay)
    torch.cuda.synchronize()
    G = G.cpu().numpy()
    r = check_logits(G, L, A, what=f"seed {seed} {fmt} n={n} k={k} m={m}")
    log(f"random shape seed={seed}: max |d|/tol = {r:.3g}")
    if fmt == "q4k":
        R = kq.gemv_staged(w_d, n, k, st, m, sc)
        torch.cuda.synchronize()
        assert np.array_equal(R.cpu().numpy(), G), "row-major weights give other logits than tiled"
        if m <= 16:
            R2 = kq.gemv_rows(w_d, n, k, x_d)
            torch.cuda.synchronize()
            assert np.array_equal(R2.cpu().numpy(), G), "kq_gemv_rows differs from the staged call"

    draft = synthetic.inject_mismatches(o_am[:m - 1], n, seed=53_000 + seed) if m > 1 else []
    if fmt == "q4k" and m <= 16:
        am, acc, lg = kq.verify(w_d, n, k, x_d, list(draft), want_logits=True)
    else:
        am, acc, lg = kq.verify_staged(wt, n, k, st, m, list(draft), sc, want_logits=True, layout=lay)
    torch.cuda.synchronize()
    am, acc = am.cpu().numpy(), acc.cpu().numpy()
    assert np.array_equal(lg.cpu().numpy(), G), "verify logits differ from the product's"
    check_argmax(am, L, A, what=f"seed {seed} verify")
    check_accept(acc[0], acc[1], draft, am, o_am, o_nc, what=f"seed {seed} verify")

    if m > 16:
        parent, token = random_tree(rng, m, o_am, n)
        tam, tacc, path, _ = kq.verify_tree_staged(wt, n, k, st, parent, token, sc, layout=lay)
        torch.cuda.synchronize()
        tam, tacc, path = tam.cpu().numpy(), tacc.cpu().numpy(), path.cpu().numpy()
        assert np.array_equal(tam, am), "tree verify argmax differs from the linear verify's"
        g_acc, g_nxt, g_path = oracle.tree_accept(parent, token, tam)
        assert (int(tacc[0]), int(tacc[1])) == (g_acc, g_nxt), "walk differs from the oracle's walk"
        assert list(path[:g_acc]) == g_path and np.all(path[g_acc:] == -1)
        if not np.any(o_nc > 0):
            assert oracle.tree_accept(parent, token, o_am)[:2] == (g_acc, g_nxt)
        log(f"random shape seed={seed}: tree of {m} nodes accepted {g_acc}")


@pytest.mark.parametrize("seed", range(24))
def test_random_chain(kq, seed):
    """3 to 6 dependent phases of random shapes (1 to 3 matrices each, Q4_K,
    rows or tiled), one launch: every logit of every matrix against the
    oracle; a second launch of the same chain gives the same bits."""
    rng = np.random.default_rng(60_000 + seed)
    m = int(rng.integers(1, 17))
    tiled = bool(rng.integers(2))
    lay = kq.LAYOUT_TILED16 if tiled else kq.LAYOUT_ROWS
    phases, expect = [], []
    for ph in range(int(rng.integers(3, 7))):
        n, k, _ = draw_shape(rng, max_m=16, n_max=40_000)
        count = int(rng.integers(1, 4))
        x = synthetic.activations(m, k, 61_000 + 10 * seed + ph)
        st = kq.stage_rows(to_dev(x))
        ws, outs = [], []
        for i in range(count):
            w = synthetic.q4k_matrix(n, k, 62_000 + 100 * seed + 10 * ph + i)
            expect.append((ph, i, n, k) + oracle.gemv_rows(w, k, x))
            wd = to_dev(w)
            ws.append(kq.tile_weights(wd, n, k) if tiled else wd)
            outs.append(torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV))
        phases.append((ws, n, k, st, outs))
    log(f"random chain seed={seed}: m={m} {'tiled' if tiled else 'rows'} phases "
        + ", ".join(f"{len(p[0])}x{p[1]}x{p[2]}" for p in phases))
    chain = kq.chain_encode(phases, m, layout=lay)
    kq.gemv_chain(chain)
    chain.status()
    torch.cuda.synchronize()
    first = [o.cpu().numpy() for p in phases for o in p[4]]
    for got, (ph, i, n, k, L, A) in zip(first, expect):
        check_logits(got, L, A, what=f"chain seed {seed} phase {ph} member {i} ({n}x{k})")
    for o in (o for p in phases for o in p[4]):
        o.fill_(float("nan"))
    kq.gemv_chain(chain)
    chain.status()
    torch.cuda.synchronize()
    again = [o.cpu().numpy() for p in phases for o in p[4]]
    assert all(np.array_equal(a, b) for a, b in zip(first, again)), "second launch differs"


@pytest.mark.parametrize("seed", range(24))
def test_random_entry_points(kq, seed):
    """The other entry points on random Q4_K shapes: a grouped launch of 1 to
    8 matrices (every logit of every member), the draft block's proposals and
    head, the verify with drafts in device memory (bitwise the host-draft
    call's result), and probability rows plus the gather on the verify's
    logits at a random temperature, with or without a soft cap."""
    from tests.test_gpu_stochastic import check_probs
    rng = np.random.default_rng(70_000 + seed)
    n, k, m = draw_shape(rng, max_m=16)
    n = max(n, 2)
    count = int(rng.integers(1, 9))
    count = max(1, min(count, MAX_WEIGHTS // (n * k)))
    tiled = bool(rng.integers(2))
    lay = kq.LAYOUT_TILED16 if tiled else kq.LAYOUT_ROWS
    log(f"random entry points seed={seed}: n={n} k={k} m={m} group of {count} ({'tiled' if tiled else 'rows'})")
    ws = [synthetic.q4k_matrix(n, k, 71_000 + 10 * seed + i) for i in range(count)]
    x = synthetic.activations(16, k, 72_000 + seed)
    wds = [to_dev(w) for w in ws]
    wus = [kq.tile_weights(wd, n, k) for wd in wds] if tiled else wds
    st = kq.stage_rows(to_dev(x[:m]))
    gs = kq.new_group_scratch(n, k, count, DEV)
    outs = kq.gemv_staged_group(wus, n, k, st, m, gs, layout=lay)
    torch.cuda.synchronize()
    for i in range(count):
        L, A = oracle.gemv_rows(ws[i], k, x[:m])
        check_logits(outs[i].cpu().numpy(), L, A, what=f"seed {seed} group member {i}")

    L16, A16 = oracle.gemv_rows(ws[0], k, x)
    vl = (3, 7, 15)[int(rng.integers(3))]
    props, head = kq.draft_block_argmax(wds[0], n, k, to_dev(x), vl, want_head=True)
    torch.cuda.synchronize()
    check_argmax(props.cpu().numpy(), L16[1:vl + 1], A16[1:vl + 1], what=f"seed {seed} draft block vl={vl}")
    check_argmax(head.cpu().numpy(), L16[:1], A16[:1], what=f"seed {seed} draft block head")

    o_am, o_nc = oracle.argmax_flags(L16[:m], A16[:m])
    draft = synthetic.inject_mismatches(o_am[:m - 1], n, seed=73_000 + seed) if m > 1 else np.zeros(0, np.int32)
    sc = kq.new_scratch(n, k, DEV)
    host = kq.verify_staged(wus[0], n, k, st, m, [int(t) for t in draft], sc, want_logits=True, layout=lay)
    on_dev = kq.verify_staged(wus[0], n, k, st, m, to_dev(np.asarray(draft, dtype=np.int32)), sc,
                              want_logits=True, layout=lay)
    torch.cuda.synchronize()
    for a, b in zip(host, on_dev):
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), "device drafts give another result"
    am, acc = host[0].cpu().numpy(), host[1].cpu().numpy()
    check_argmax(am, L16[:m], A16[:m], what=f"seed {seed} verify")
    check_accept(acc[0], acc[1], draft, am, o_am, o_nc, what=f"seed {seed} verify")

    lg = host[2]
    lh = lg.cpu().numpy()
    temperature = max(1e-3, float(np.std(lh)) * float(rng.uniform(0.2, 2.0)))
    cap = 0.0 if rng.random() < 0.5 else float(np.abs(lh).max()) * float(rng.uniform(0.3, 1.0))
    P = kq.softmax_rows(lg, temperature, cap)
    torch.cuda.synchronize()
    ph = P.cpu().numpy()
    r = check_probs(ph, lh, temperature, cap, f"seed {seed} rows T={temperature:.3g} cap={cap:.3g}")
    log(f"random entry points seed={seed}: probability rows max err / tol = {r:.3g}")
    tok = rng.integers(0, n, m).astype(np.int32)
    got = kq.gather_rows(P, to_dev(tok)).cpu().numpy()
    assert np.array_equal(got, ph[np.arange(m), tok]), "gather differs from indexing the rows"
