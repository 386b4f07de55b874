"""GPU parity tests: the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs of every workload shape, plus edge
shapes, planted ties, row invariance, determinism and the staged API."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_accept, check_argmax, check_logits, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


DEV = "cuda:0"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_logits(kq, w_d, n, k, x):
    out = kq.gemv_rows(w_d, n, k, to_dev(x))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_verify(kq, w_d, n, k, x, draft, want_logits=False):
    am, acc, lg = kq.verify(w_d, n, k, to_dev(x), list(draft), want_logits=want_logits)
    torch.cuda.synchronize()
    return am.cpu().numpy(), acc.cpu().numpy(), (lg.cpu().numpy() if lg is not None else None)


def test_tiny_config_verify_all_accept_lengths(kq):
    c = synthetic.TINY
    n, k, m = c["n"], c["k"], c["m"]
    log(f"tiny: n={n} k={k} m={m}")
    w = synthetic.q4k_matrix(n, k, c["seed"])
    x = synthetic.activations(m, k, c["seed"])
    L, A = oracle.gemv_rows(w, k, x)
    w_d = to_dev(w)
    G = gpu_logits(kq, w_d, n, k, x)
    ratio = check_logits(G, L, A, what="tiny")
    log(f"tiny: max |d|/tol = {ratio:.3g}")
    o_am, o_nc = oracle.argmax_flags(L, A)
    drafts = [synthetic.forced_draft(o_am[:m - 1], a, n) for a in range(m)]
    drafts += [synthetic.inject_mismatches(o_am[:m - 1], n, seed=1000 + t) for t in range(16)]
    seen = set()
    for i, d in enumerate(drafts):
        g_am, g_acc, g_lg = gpu_verify(kq, w_d, n, k, x, d, want_logits=(i == 0))
        check_argmax(g_am, L, A, what=f"tiny trial {i}")
        acc_o, _ = check_accept(g_acc[0], g_acc[1], d, g_am, o_am, o_nc, what=f"tiny trial {i}")
        seen.add(int(g_acc[0]))
        if g_lg is not None:
            assert np.array_equal(g_lg, G), "verify logits differ from gemv logits"
    assert seen >= set(range(m)), f"accepted lengths seen: {sorted(seen)}"


def test_square_m_sweep_row_invariance(kq):
    c = synthetic.SQUARE
    n = k = c["n"]
    log(f"square: n=k={n}")
    w = synthetic.q4k_matrix(n, k, c["seed"])
    x = synthetic.activations(16, k, c["seed"])
    L, A = oracle.gemv_rows(w, k, x)
    w_d = to_dev(w)
    G16 = gpu_logits(kq, w_d, n, k, x)
    check_logits(G16, L, A, what="square m=16")
    for mm in c["ms"]:
        Gm = gpu_logits(kq, w_d, n, k, x[:mm])
        check_logits(Gm, L[:mm], A[:mm], what=f"square m={mm}")
        assert np.array_equal(Gm, G16[:mm]), f"rows of m={mm} call differ from m=16 call"
    for i in (0, 7, 15):  # row i of the 16-row call equals the 1-row call on x[i]
        G1 = gpu_logits(kq, w_d, n, k, x[i:i + 1])
        assert np.array_equal(G1[0], G16[i])
    log("square: ok")


def test_fc_projection(kq):
    c = synthetic.FC
    n, k, m = c["n"], c["k"], c["m"]
    log(f"fc: n={n} k={k} m={m}")
    w = synthetic.q4k_matrix(n, k, c["seed"])
    x = synthetic.fc_activations(m, c["seed"])
    L, A = oracle.gemv_rows(w, k, x)
    G = gpu_logits(kq, to_dev(w), n, k, x)
    ratio = check_logits(G, L, A, what="fc")
    log(f"fc: max |d|/tol = {ratio:.3g}")


def test_lm_head_verify_full_size(kq):
    c = synthetic.LM_HEAD
    n, k, m = c["n"], c["k"], c["m"]
    log(f"lm head: n={n} k={k} m={m} (oracle over all rows)")
    w = synthetic.q4k_matrix(n, k, c["seed"])
    x = synthetic.activations(m, k, c["seed"])
    L, A = oracle.gemv_rows(w, k, x)
    o_am, o_nc = oracle.argmax_flags(L, A)
    log(f"lm head: oracle flagged rows {int(np.sum(o_nc > 0))}")
    w_d = to_dev(w)
    drafts = [synthetic.forced_draft(o_am[:m - 1], a, n) for a in (0, 1, 7, 15)]
    drafts += [synthetic.inject_mismatches(o_am[:m - 1], n, seed=1000 + t) for t in range(8)]
    for i, d in enumerate(drafts):
        g_am, g_acc, g_lg = gpu_verify(kq, w_d, n, k, x, d, want_logits=(i == 0))
        if g_lg is not None:
            ratio = check_logits(g_lg, L, A, what="lm head")
            log(f"lm head: max |d|/tol = {ratio:.3g}")
        check_argmax(g_am, L, A, what=f"lm head trial {i}")
        check_accept(g_acc[0], g_acc[1], d, g_am, o_am, o_nc, what=f"lm head trial {i}")
    log("lm head: ok")
    # The same 16-row block as a draft block: proposals are the argmax of rows
    # 1..verify_length, the head is row 0's (row-major and tiled weights, the
    # full block and exactly verify_length + 1 rows).
    x_d = to_dev(x)
    wt = kq.tile_weights(w_d, n, k)
    scratch = kq.new_scratch(n, k, DEV)
    for vl in kq.DRAFT_VERIFY_LENGTHS:
        props, head = kq.draft_block_argmax(w_d, n, k, x_d, vl, want_head=True)
        props_short, _ = kq.draft_block_argmax(w_d, n, k, x_d[:vl + 1].contiguous(), vl)
        st = kq.stage_rows(x_d[:vl + 1].contiguous())
        props_t, head_t = kq.draft_block_argmax_staged(wt, n, k, st, vl, scratch, want_head=True,
                                                       layout=kq.LAYOUT_TILED16)
        torch.cuda.synchronize()
        p, h = props.cpu().numpy(), head.cpu().numpy()
        assert p.shape == (vl,)
        check_argmax(p, L[1:vl + 1], A[1:vl + 1], what=f"draft block proposals vl={vl}")
        check_argmax(h, L[:1], A[:1], what=f"draft block head vl={vl}")
        assert np.array_equal(p, props_short.cpu().numpy())
        assert np.array_equal(p, props_t.cpu().numpy()) and np.array_equal(h, head_t.cpu().numpy())
    log("draft block proposals: ok")


@pytest.mark.parametrize("shape", [(6656, 6656), (17920, 6656), (6656, 17920)])
def test_stack_shapes_sampled_rows(kq, shape):
    n, k = shape
    log(f"stack shape n={n} k={k}")
    g = [s for s in synthetic.stack_matrices(1) if (s.n, s.k) == shape][0]
    w = synthetic.q4k_matrix(n, k, g.seed)
    x = synthetic.activations(16, k, synthetic.stack_activation_seed(k))
    rng = np.random.default_rng(n + k)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, n - 17, n - 1], rng.integers(0, n, 250)]))
    L, A = oracle.gemv_rows(w, k, x, rows=rows)
    w_d = to_dev(w)
    staged = kq.stage_rows(to_dev(x))
    scratch = kq.new_scratch(n, k, DEV)
    for mm in (1, 16):
        st = staged if mm == 16 else kq.stage_rows(to_dev(x[:1]))
        G = kq.gemv_staged(w_d, n, k, st, mm, scratch)
        torch.cuda.synchronize()
        check_logits(G.cpu().numpy()[:, rows], L[:mm], A[:mm], what=f"stack {shape} m={mm}")


@pytest.mark.parametrize("n,k,count", [(6656, 6656, 3), (17920, 6656, 2)])
def test_stack_grouped_launches_sampled_rows(kq, n, k, count):
    """The stack's grouped launches (q,k,v and gate,up) at full size, in the
    launch configuration bench.py times: tiled weights, one launch per group."""
    log(f"stack group {count} x n={n} k={k}")
    mats = [s for s in synthetic.stack_matrices(1) if (s.n, s.k) == (n, k)][:count]
    assert len(mats) == count
    ws = [synthetic.q4k_matrix(n, k, g.seed) for g in mats]
    x = synthetic.activations(16, k, synthetic.stack_activation_seed(k))
    rng = np.random.default_rng(n + 7 * k + count)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 127, 128, 191, 192, n - 17, n - 1], rng.integers(0, n, 100)]))
    wts = [kq.tile_weights(to_dev(w), n, k) for w in ws]
    gs = kq.new_group_scratch(n, k, count, DEV)
    for mm in (16, 1):
        st = kq.stage_rows(to_dev(x[:mm]))
        outs = kq.gemv_staged_group(wts, n, k, st, mm, gs, layout=kq.LAYOUT_TILED16)
        torch.cuda.synchronize()
        for i in range(count):
            L, A = oracle.gemv_rows(ws[i], k, x[:mm], rows=rows)
            check_logits(outs[i].cpu().numpy()[:, rows], L, A, what=f"group {n}x{k} member {i} m={mm}")


EDGE = [(1, 256), (17, 256), (16, 512), (129, 1280), (1000, 2304), (513, 3328), (2048, 9216)]


@pytest.mark.parametrize("n,k", EDGE)
def test_edge_shapes(kq, n, k):
    log(f"edge n={n} k={k}")
    w = synthetic.q4k_matrix(n, k, 7 + n + k)
    x = synthetic.activations(16, k, 9 + n + k)
    L, A = oracle.gemv_rows(w, k, x)
    w_d = to_dev(w)
    for mm in (1, 3, 16):
        G = gpu_logits(kq, w_d, n, k, x[:mm])
        check_logits(G, L[:mm], A[:mm], what=f"edge {n}x{k} m={mm}")
        o_am, o_nc = oracle.argmax_flags(L[:mm], A[:mm])
        d = synthetic.inject_mismatches(o_am[:mm - 1], n, seed=n * 31 + mm) if mm > 1 else []
        g_am, g_acc, _ = gpu_verify(kq, w_d, n, k, x[:mm], d)
        check_argmax(g_am, L[:mm], A[:mm], what=f"edge {n}x{k} m={mm}")
        check_accept(g_acc[0], g_acc[1], d, g_am, o_am, o_nc, what=f"edge {n}x{k} m={mm}")


@pytest.mark.parametrize("n,k", [(2000, 1024), (513, 3328)])
def test_draft_block_small(kq, n, k):
    log(f"draft block n={n} k={k}")
    w = synthetic.q4k_matrix(n, k, 61 + n)
    # duplicate row 7 at row 700 (or the last row): an exact tie, the lowest
    # index must win wherever it is the maximum
    w = w.copy()
    w[min(700, n - 1)] = w[7]
    x = synthetic.activations(16, k, 62 + n)
    L, A = oracle.gemv_rows(w, k, x)
    w_d, x_d = to_dev(w), to_dev(x)
    for vl in kq.DRAFT_VERIFY_LENGTHS:
        props, head = kq.draft_block_argmax(w_d, n, k, x_d, vl, want_head=True)
        torch.cuda.synchronize()
        check_argmax(props.cpu().numpy(), L[1:vl + 1], A[1:vl + 1], what=f"draft {n}x{k} vl={vl}")
        check_argmax(head.cpu().numpy(), L[:1], A[:1], what=f"draft head {n}x{k} vl={vl}")


def test_stream_probe_reads_every_byte(kq):
    # the XOR of the per-workgroup words is the XOR of every 32-bit word
    rng = np.random.default_rng(5)
    for nbytes in (16, 3 * (1 << 20) + 16, 8192 * 1024 * 16 + 48):
        a = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
        sink = kq.stream_probe(to_dev(a.view(np.uint8)))
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert int(got) == int(np.bitwise_xor.reduce(a)), nbytes


def test_one_hot_rows_extract_weights(kq):
    n, k = 300, 2048
    w = synthetic.q4k_matrix(n, k, 41)
    Wd = oracle.decode_matrix(w, k)
    cols = [0, 31, 32, 255, 256, 1023, 1024, 2047, 100, 600, 1500, 1999, 64, 96, 128, 160]
    x = np.zeros((16, k), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    G = gpu_logits(kq, to_dev(w), n, k, x)
    for i, c in enumerate(cols):
        # d*sc*q and dmin*m are exact in fp32, so one rounding of their difference
        assert np.all(np.abs(G[i] - Wd[:, c]) <= 2.0 ** -24 * np.abs(Wd[:, c])), c


def test_planted_exact_ties_pick_lowest_index(kq):
    n, k = 700, 1024
    w = synthetic.q4k_matrix(n, k, 51)
    x = synthetic.activations(1, k, 52)
    L, A = oracle.gemv_rows(w, k, x)
    o_am, _ = oracle.argmax_flags(L, A)
    b = int(o_am[0])
    p = 5 if b != 5 else 6
    q = n - 3 if b != n - 3 else n - 4
    w2 = w.copy()
    w2[p] = w[b]  # identical weight rows: an exact three-way tie for the maximum
    w2[q] = w[b]
    w2_d = to_dev(w2)
    G = gpu_logits(kq, w2_d, n, k, x)
    assert G[0, p] == G[0, b] == G[0, q]
    g_am, g_acc, _ = gpu_verify(kq, w2_d, n, k, x, [])
    assert int(g_am[0]) == min(p, q, b)
    assert int(g_acc[0]) == 0 and int(g_acc[1]) == min(p, q, b)


def test_deterministic_and_staged_equals_all_in_one(kq):
    n, k = 3000, 6656
    w = synthetic.q4k_matrix(n, k, 61)
    x = synthetic.activations(16, k, 62)
    w_d, x_d = to_dev(w), to_dev(x)
    a = kq.gemv_rows(w_d, n, k, x_d).cpu().numpy()
    b = kq.gemv_rows(w_d, n, k, x_d).cpu().numpy()
    assert np.array_equal(a, b)
    st = kq.stage_rows(x_d)
    sc = kq.new_scratch(n, k, DEV)
    c = kq.gemv_staged(w_d, n, k, st, 16, sc).cpu().numpy()
    assert np.array_equal(a, c)
    d = list(range(15))
    am1, acc1, _ = kq.verify(w_d, n, k, x_d, d)
    am2, acc2, lg2 = kq.verify_staged(w_d, n, k, st, 16, d, sc, want_logits=True)
    assert np.array_equal(am1.cpu().numpy(), am2.cpu().numpy())
    assert np.array_equal(acc1.cpu().numpy(), acc2.cpu().numpy())
    assert np.array_equal(lg2.cpu().numpy(), a)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        e = kq.gemv_rows(w_d, n, k, x_d)
    s.synchronize()
    assert np.array_equal(e.cpu().numpy(), a)


def test_activation_range_scaling(kq):
    n, k = 256, 2048
    w = synthetic.q4k_matrix(n, k, 71)
    base = synthetic.activations(16, k, 72)
    scales = np.array([1e-30, 1e-8, 1e-4, 1.0, 1e4, 1e8, 1e20, 3e30] * 2, dtype=np.float64)
    x = (base * scales[:, None]).astype(np.float32)
    L, A = oracle.gemv_rows(w, k, x)
    G = gpu_logits(kq, to_dev(w), n, k, x)
    check_logits(G, L, A, what="activation range")


def test_grouped_launch(kq):
    n, k, count = 2000, 6656, 3
    log(f"grouped launch: {count} x n={n} k={k}")
    ws = [synthetic.q4k_matrix(n, k, 80 + i) for i in range(count)]
    x = synthetic.activations(16, k, 85)
    rows = np.array([0, 1, 15, 16, 777, n - 17, n - 1])
    ws_d = [to_dev(w) for w in ws]
    st = kq.stage_rows(to_dev(x))
    gs = kq.new_group_scratch(n, k, count, DEV)
    for mm in (16, 5):
        st_m = st if mm == 16 else kq.stage_rows(to_dev(x[:mm]))
        outs = kq.gemv_staged_group(ws_d, n, k, st_m, mm, gs)
        again = kq.gemv_staged_group(ws_d, n, k, st_m, mm, gs)
        torch.cuda.synchronize()
        for i in range(count):
            G = outs[i].cpu().numpy()
            assert np.array_equal(G, again[i].cpu().numpy())
            L, A = oracle.gemv_rows(ws[i], k, x[:mm], rows=rows)
            check_logits(G[:, rows], L, A, what=f"group member {i} m={mm}")


def tile_reference(w_bytes, n, k):
    """The tiled layout written out from its definition in kq.h, in numpy:
    record (b, t) of 2,304 bytes at (b * tiles + t) * 2,304 holds the 16
    headers of tile t's rows, then quant bytes [16g, 16g+16) of row r at
    256 + 16 (16g + r), then quant bytes [64+16g, 80+16g) at 1,280 + ..."""
    kb, nt = k // 256, -(-n // 16)
    pad = np.zeros((nt * 16, kb, 144), np.uint8)
    pad[:n] = w_bytes.reshape(n, kb, 144)
    t = pad.reshape(nt, 16, kb, 144).transpose(2, 0, 1, 3)  # [b][tile][row][144]
    out = np.zeros((kb, nt, 2304), np.uint8)
    out[:, :, :256] = t[:, :, :, :16].reshape(kb, nt, 256)
    for half, base in ((0, 256), (1, 1280)):
        q = t[:, :, :, 16 + 64 * half:80 + 64 * half].reshape(kb, nt, 16, 4, 16)  # [b][tile][row][g][16]
        out[:, :, base:base + 1024] = q.transpose(0, 1, 3, 2, 4).reshape(kb, nt, 1024)
    return out.reshape(-1)


def test_tile_weights_matches_layout_definition(kq):
    for n, k in [(37, 512), (16, 256), (1000, 2304)]:
        w = synthetic.q4k_matrix(n, k, 90 + n)
        got = kq.tile_weights(to_dev(w), n, k).cpu().numpy()
        assert got.size == kq.tiled_bytes(n, k)
        assert np.array_equal(got, tile_reference(w, n, k)), (n, k)


@pytest.mark.parametrize("n,k,m", [(512, 1024, 4), (17, 256, 16), (129, 1280, 16), (1000, 2304, 7),
                                   (6656, 6656, 16), (2048, 9216, 16), (6656, 17920, 1)])
def test_tiled_layout_bitwise_equal_to_rows(kq, n, k, m):
    log(f"tiled vs rows: n={n} k={k} m={m}")
    w = synthetic.q4k_matrix(n, k, 100 + n + k)
    x = synthetic.activations(m, k, 101)
    w_d = to_dev(w)
    wt = kq.tile_weights(w_d, n, k)
    st = kq.stage_rows(to_dev(x))
    sc = kq.new_scratch(n, k, DEV)
    a = kq.gemv_staged(w_d, n, k, st, m, sc).cpu().numpy()
    b = kq.gemv_staged(wt, n, k, st, m, sc, layout=kq.LAYOUT_TILED16).cpu().numpy()
    assert np.array_equal(a, b)
    rows = np.unique(np.array([0, 1, 15, 16, n // 2, n - 1]))
    L, A = oracle.gemv_rows(w, k, x, rows=rows)
    check_logits(b[:, rows], L, A, what=f"tiled n={n} k={k}")


def test_tiled_lm_head_verify_and_group(kq):
    h = synthetic.LM_HEAD
    n, k = h["n"], h["k"]
    w = synthetic.q4k_matrix(n, k, h["seed"])
    x = synthetic.activations(16, k, 7)
    w_d = to_dev(w)
    wt = kq.tile_weights(w_d, n, k)
    st = kq.stage_rows(to_dev(x))
    sc = kq.new_scratch(n, k, DEV)
    d = [int(t) for t in np.random.default_rng(3).integers(0, n, 15)]
    r = kq.verify_staged(w_d, n, k, st, 16, d, sc, want_logits=True)
    t = kq.verify_staged(wt, n, k, st, 16, d, sc, want_logits=True, layout=kq.LAYOUT_TILED16)
    for u, v in zip(r, t):
        assert np.array_equal(u.cpu().numpy(), v.cpu().numpy())
    del w_d, wt
    n2, k2, count = 2000, 6656, 3
    ws = [synthetic.q4k_matrix(n2, k2, 80 + i) for i in range(count)]
    ws_d = [to_dev(v) for v in ws]
    wts = [kq.tile_weights(v, n2, k2) for v in ws_d]
    st2 = kq.stage_rows(to_dev(synthetic.activations(16, k2, 85)))
    gs = kq.new_group_scratch(n2, k2, count, DEV)
    a = kq.gemv_staged_group(ws_d, n2, k2, st2, 16, gs)
    b = kq.gemv_staged_group(wts, n2, k2, st2, 16, gs, layout=kq.LAYOUT_TILED16)
    for u, v in zip(a, b):
        assert np.array_equal(u.cpu().numpy(), v.cpu().numpy())


def test_device_drafts_and_draft_block_to_verify_on_device(kq):
    """Draft tokens in device memory (kq_verify_staged_dev) give the host
    path's result; tokens outside [0, n) count as mismatches; the draft
    block's proposals (device) feed the verify with no host round trip."""
    n, k, m = 3000, 2304, 16
    w = synthetic.q4k_matrix(n, k, 61)
    x = synthetic.activations(m, k, 62)
    L, A = oracle.gemv_rows(w, k, x)
    o_am, o_nc = oracle.argmax_flags(L, A)
    wt = kq.tile_weights(to_dev(w), n, k)
    st = kq.stage_rows(to_dev(x))
    sc = kq.new_scratch(n, k, DEV)
    rng = np.random.default_rng(63)
    for trial in range(6):
        d = [int(t) for t in synthetic.forced_draft(o_am[:m - 1], int(rng.integers(0, m)), n)]
        am_h, acc_h, _ = kq.verify_staged(wt, n, k, st, m, d, sc, layout=kq.LAYOUT_TILED16)
        acc_h = acc_h.cpu().numpy().copy()
        dd = torch.tensor(d, dtype=torch.int32, device=DEV)
        am_d, acc_d, _ = kq.verify_staged(wt, n, k, st, m, dd, sc, layout=kq.LAYOUT_TILED16)
        torch.cuda.synchronize()
        assert np.array_equal(am_h.cpu().numpy(), am_d.cpu().numpy())
        assert np.array_equal(acc_h, acc_d.cpu().numpy()), trial
        check_accept(acc_d.cpu().numpy()[0], acc_d.cpu().numpy()[1], d, am_d.cpu().numpy(), o_am, o_nc,
                     what=f"device drafts trial {trial}")
    # out-of-range device tokens are mismatches (compared, never used as an index)
    for bad in (-1, n, n + 1000, -(1 << 30)):
        d = [int(t) for t in o_am[:m - 1]]
        d[5] = bad
        am_d, acc_d, _ = kq.verify_staged(wt, n, k, st, m, torch.tensor(d, dtype=torch.int32, device=DEV), sc,
                                          layout=kq.LAYOUT_TILED16)
        torch.cuda.synchronize()
        am_d = am_d.cpu().numpy()
        assert tuple(acc_d.cpu().numpy()) == oracle.accept(d, am_d)
    # draft block -> verify on one stream: the proposals of a 16-row block
    # (rows 1..15) verified as the draft of the same block: all accepted
    props, head = kq.draft_block_argmax_staged(wt, n, k, st, 15, sc, want_head=True, layout=kq.LAYOUT_TILED16)
    am_b = torch.empty(16, dtype=torch.int32, device=DEV)
    acc_b = torch.empty(2, dtype=torch.int32, device=DEV)
    shifted = torch.empty(15, dtype=torch.int32, device=DEV)
    shifted[0] = head[0]
    shifted[1:] = props[:14]
    kq.verify_staged(wt, n, k, st, 16, shifted, sc, out=(am_b, acc_b, None), layout=kq.LAYOUT_TILED16)
    torch.cuda.synchronize()
    a = am_b.cpu().numpy()
    assert tuple(acc_b.cpu().numpy()) == (15, int(a[15]))
    assert np.array_equal(a[1:16], props.cpu().numpy()) and int(a[0]) == int(head.cpu().numpy()[0])


def test_degenerate_inputs(kq):
    """The method's degenerate ends, Q4_K on both layouts and through the
    verify:
    * blocks at the ends of every field: fp16 d and dmin subnormal (down to
      2^-24), tiny normal, or the largest finite value 65504; 6-bit scales
      and mins 0 and 63; nibbles 0 and 15;
    * all-zero activation rows among ordinary ones: every logit of such a
      row is exactly zero, so its argmax is index 0 (all indices tie, the
      lowest wins) and the row is flagged;
    * an all-zero weight matrix: every logit zero, every argmax 0."""
    from tests.q4k_pack import pack_block
    g = np.random.default_rng(9)
    n, k = 200, 1024
    d_choices = [0x0001, 0x0003, 0x03FF, 0x0400, 0x1000, 0x2A00, 0x7BFF]  # 2^-24 ... 65504
    rows = []
    for r in range(n):
        blocks = []
        for b in range(k // 256):
            d, dm = int(g.choice(d_choices)), int(g.choice(d_choices))
            sc = g.choice([0, 63, 1, 62], 8)
            mn = g.choice([0, 63, 1], 8)
            q = g.choice([0, 15, 1, 14], 256)
            blocks.append(pack_block(d, dm, sc, mn, q))
        rows.append(b"".join(blocks))
    w = np.frombuffer(b"".join(rows), dtype=np.uint8).reshape(n, -1).copy()
    x = synthetic.activations(16, k, 91)
    x[3] = 0.0
    x[9] = 0.0
    L, A = oracle.gemv_rows(w, k, x)
    assert not np.any(L[3]) and not np.any(L[9])
    w_d = to_dev(w)
    G = gpu_logits(kq, w_d, n, k, x)
    r = check_logits(G, L, A, what="degenerate fields")
    log(f"degenerate fields: max |d|/tol = {r:.3g}")
    assert not np.any(G[3]) and not np.any(G[9]), "an all-zero activation row gave a non-zero logit"
    wt = kq.tile_weights(w_d, n, k)
    sc_ = kq.new_scratch(n, k, DEV)
    T = kq.gemv_staged(wt, n, k, kq.stage_rows(to_dev(x)), 16, sc_, layout=kq.LAYOUT_TILED16)
    torch.cuda.synchronize()
    assert np.array_equal(T.cpu().numpy(), G)
    o_am, o_nc = oracle.argmax_flags(L, A)
    d = synthetic.inject_mismatches(o_am[:15], n, seed=92)
    g_am, g_acc, _ = gpu_verify(kq, w_d, n, k, x, d)
    check_argmax(g_am, L, A, what="degenerate fields")
    check_accept(g_acc[0], g_acc[1], d, g_am, o_am, o_nc, what="degenerate fields")
    assert int(g_am[3]) == 0 and int(g_am[9]) == 0 and o_nc[3] == n - 1

    z = np.zeros_like(w)
    G0 = gpu_logits(kq, to_dev(z), n, k, x)
    assert not np.any(G0), "an all-zero matrix gave a non-zero logit"
    z_am, z_acc, _ = gpu_verify(kq, to_dev(z), n, k, x, [0] * 15)
    assert not np.any(z_am) and (int(z_acc[0]), int(z_acc[1])) == (15, 0)
