"""GPU parity of the Q5_K and Q6_K paths (tiled copies from llama.cpp rows,
the same staged activations and kernel structure as Q4_K) against the
oracle's fp64 products: every logit on ragged shapes, exact weight columns
from one-hot rows, row invariance, grouped launches, and the Q6_K LM-head
verify (argmax and accept) at full size."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_accept, check_argmax, check_logits, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FMTS = ["q5k", "q6k"]


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_gemv(kq, fmt, w, n, k, x, scratch=None):
    """Logits [m, n] through kq_tile_weights_fmt + kq_stage_rows + kq_gemv_staged."""
    wt = kq.tile_weights(to_dev(w), n, k, fmt=fmt)
    st = kq.stage_rows(to_dev(x))
    sc = scratch if scratch is not None else kq.new_scratch(n, k, DEV)
    out = kq.gemv_staged(wt, n, k, st, x.shape[0], sc, layout=kq.FORMATS[fmt][0])
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 256), (17, 512), (300, 1024), (1000, 2304), (129, 6656), (2049, 768)])
def test_ragged_shapes_every_logit(kq, fmt, n, k):
    w = synthetic.kquant_matrix(fmt, n, k, 500 + n)
    x = synthetic.activations(16, k, 600 + k)
    for m in (16, 3, 1):
        log(f"{fmt} n={n} k={k} m={m}")
        L, A = oracle.gemv_rows(w, k, x[:m], fmt=fmt)
        G = gpu_gemv(kq, fmt, w, n, k, x[:m])
        r = check_logits(G, L, A, what=f"{fmt} n={n} k={k} m={m}")
        log(f"{fmt} n={n} k={k} m={m}: max |d|/tol = {r:.3g}")


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_rows_extract_weights(kq, fmt):
    """x = e_c returns weight column c. Q6_K: d sc (q - 32) is exact in fp32,
    so the column is bit-exact; Q5_K: d sc q and dmin m are exact, one
    rounding of their difference."""
    n, k = 300, 2048
    w = synthetic.kquant_matrix(fmt, n, k, 41)
    Wd = oracle.decode_matrix(w, k, fmt)
    cols = [0, 15, 16, 31, 32, 255, 256, 1023, 1024, 2047, 100, 600, 1500, 1999, 64, 96]
    x = np.zeros((16, k), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    G = gpu_gemv(kq, fmt, w, n, k, x)
    for i, c in enumerate(cols):
        if fmt == "q6k":
            assert np.array_equal(G[i].astype(np.float64), Wd[:, c]), c
        else:
            assert np.all(np.abs(G[i] - Wd[:, c]) <= 2.0 ** -24 * np.abs(Wd[:, c])), c


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_rows_at_lm_head_shape(kq, fmt):
    """One-hot rows at the LM head's shape (131,072 rows: two tiles per
    wave): every weight column bit-exact for Q6_K (one rounding for Q5_K).
    A stale or wrong operand remainder in any tile shows here even when the
    logits stay inside the tolerance."""
    h = synthetic.LM_HEAD
    n, k = h["n"], h["k"]
    w = synthetic.kquant_matrix(fmt, n, k, 57)
    cols = [0, 15, 16, 31, 255, 256, 1000, 2047, 3333, 4096, 5000, 6000, 6400, 6655, 100, 777]
    x = np.zeros((16, k), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    W, _ = oracle.gemv_rows(w, k, x, fmt=fmt)  # exact columns (fp64 products of exact weights by 1)
    G = gpu_gemv(kq, fmt, w, n, k, x)
    for i, c in enumerate(cols):
        if fmt == "q6k":
            bad = np.nonzero(G[i].astype(np.float64) != W[i])[0]
            assert bad.size == 0, f"column {c}: {bad.size} rows differ, first {bad[:5]}"
        else:
            assert np.all(np.abs(G[i] - W[i]) <= 2.0 ** -24 * np.abs(W[i])), c


@pytest.mark.parametrize("fmt", FMTS)
def test_extreme_fields(kq, fmt):
    """Blocks at the ends of every field's range: Q6_K scales -128 and 127
    with q = 0 and 63 (|sc (q - 32)| up to 4,096, the products that need the
    split B operand); Q5_K scales and mins 63 with q = 31."""
    from tests.q4k_pack import f16_bits, pack_q5k_block, pack_q6k_block
    g = np.random.default_rng(5)
    n, k = 64, 512
    rows = []
    for r in range(n):
        blocks = []
        for b in range(k // 256):
            if fmt == "q6k":
                sc = g.choice([-128, 127, -127, 1, -1, 0, 99], 16)
                q = g.choice([0, 63, 1, 62, 32, 31], 256)
                blocks.append(pack_q6k_block(f16_bits(float(np.float16(g.uniform(0.0002, 0.01)))), sc, q))
            else:
                sc = g.choice([63, 62, 1, 0], 8)
                mn = g.choice([63, 0, 1], 8)
                q = g.choice([31, 0, 16, 15], 256)
                blocks.append(pack_q5k_block(f16_bits(float(np.float16(g.uniform(0.001, 0.05)))),
                                             f16_bits(float(np.float16(g.uniform(0.001, 0.05)))), sc, mn, q))
        rows.append(b"".join(blocks))
    w = np.frombuffer(b"".join(rows), dtype=np.uint8).reshape(n, -1).copy()
    x = synthetic.activations(16, k, 77)
    L, A = oracle.gemv_rows(w, k, x, fmt=fmt)
    G = gpu_gemv(kq, fmt, w, n, k, x)
    r = check_logits(G, L, A, what=f"{fmt} extremes")
    log(f"{fmt} extremes: max |d|/tol = {r:.3g}")


@pytest.mark.parametrize("fmt", FMTS)
def test_row_invariance_determinism_and_groups(kq, fmt):
    """Row 0 of an M = 16 call is bitwise the M = 1 call; repeats are
    bitwise equal; a grouped launch of three matrices matches the oracle on
    sampled rows."""
    n, k = 2000, 6656
    ws = [synthetic.kquant_matrix(fmt, n, k, 80 + i) for i in range(3)]
    x = synthetic.activations(16, k, 85)
    wts = [kq.tile_weights(to_dev(w), n, k, fmt=fmt) for w in ws]
    lay = kq.FORMATS[fmt][0]
    st16 = kq.stage_rows(to_dev(x))
    st1 = kq.stage_rows(to_dev(x[:1]))
    sc = kq.new_scratch(n, k, DEV)
    a = kq.gemv_staged(wts[0], n, k, st16, 16, sc, layout=lay).cpu().numpy()
    b = kq.gemv_staged(wts[0], n, k, st16, 16, sc, layout=lay).cpu().numpy()
    c = kq.gemv_staged(wts[0], n, k, st1, 1, sc, layout=lay).cpu().numpy()
    assert np.array_equal(a, b), "not deterministic"
    assert np.array_equal(a[0], c[0]), "row 0 depends on m"
    rows = np.array([0, 1, 15, 16, 999, 1999])
    L, A = oracle.gemv_rows(ws[0], k, x, rows=rows, fmt=fmt)
    check_logits(a[:, rows], L, A, what=f"{fmt} 2000x6656")
    gs = kq.new_group_scratch(n, k, 3, DEV)
    grp = kq.gemv_staged_group(wts, n, k, st16, 16, gs, layout=lay)
    torch.cuda.synchronize()
    for i, r in enumerate(grp):
        r = r.cpu().numpy()
        L, A = oracle.gemv_rows(ws[i], k, x, rows=rows, fmt=fmt)
        check_logits(r[:, rows], L, A, what=f"{fmt} group member {i}")


def test_q6k_lm_head_verify_full_size(kq):
    """The LM head as Q6_K (the output layer's usual k-quant) at 6,656 ->
    131,072, 16 rows: logits of every row against the oracle, argmax with
    flags, and the accept rule for injected drafts; the draft block's
    proposals from the same weights equal the verify's argmax rows."""
    c = synthetic.LM_HEAD
    n, k, m = c["n"], c["k"], c["m"]
    log(f"q6k lm head: n={n} k={k} m={m} (oracle over all rows)")
    w = synthetic.q6k_matrix(n, k, c["seed"])
    x = synthetic.activations(m, k, c["seed"])
    L, A = oracle.gemv_rows(w, k, x, fmt="q6k")
    o_am, o_nc = oracle.argmax_flags(L, A)
    log(f"q6k lm head: oracle flagged rows {int(np.sum(o_nc > 0))}")
    wt = kq.tile_weights(to_dev(w), n, k, fmt="q6k")
    st = kq.stage_rows(to_dev(x))
    sc = kq.new_scratch(n, k, DEV)
    lay = kq.LAYOUT_Q6K_TILED16
    drafts = [synthetic.forced_draft(o_am[:m - 1], a, n) for a in (0, 7, 15)]
    drafts += [synthetic.inject_mismatches(o_am[:m - 1], n, seed=2000 + t) for t in range(4)]
    for i, d in enumerate(drafts):
        am, acc, lg = kq.verify_staged(wt, n, k, st, m, d, sc, want_logits=(i == 0), layout=lay)
        torch.cuda.synchronize()
        am, acc = am.cpu().numpy(), acc.cpu().numpy()
        if lg is not None:
            r = check_logits(lg.cpu().numpy(), L, A, what="q6k lm head")
            log(f"q6k lm head: max |d|/tol = {r:.3g}")
        check_argmax(am, L, A, what=f"q6k lm head trial {i}")
        check_accept(acc[0], acc[1], d, am, o_am, o_nc, what=f"q6k lm head trial {i}")
    props, head = kq.draft_block_argmax_staged(wt, n, k, st, 15, sc, want_head=True, layout=lay)
    torch.cuda.synchronize()
    assert np.array_equal(props.cpu().numpy(), am[1:16]) and int(head.cpu().numpy()[0]) == int(am[0])
    log("q6k lm head: ok")
