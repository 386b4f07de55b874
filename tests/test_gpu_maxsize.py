"""GPU parity at the largest shapes the boundary accepts.

The kernels address a weight matrix and a staged activation block with
32-bit byte offsets, so each must stay below 4 GiB (the shape rule every
entry point checks). These tests run each row-group geometry on a weight
matrix just under that limit, and one matrix whose staged activations are
just under it (K = 64,829,440: a single 128-row group split over every
workgroup). Every logit is compared with the oracle, argmax and accept over
all rows, and the tiled layout, the verify and a one-phase chain are checked
against the row-major product."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_accept, check_argmax, check_logits, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LIMIT = 1 << 32


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_all(kq, n, k, m, seed, threads=0):
    """Row-major product, verify, tiled product and a one-phase chain on one
    seeded matrix, each against the oracle's fp64 logits of every row."""
    w = synthetic.q4k_matrix(n, k, seed)
    x = synthetic.activations(m, k, seed + 1)
    log(f"max size n={n} k={k} m={m}: oracle over all rows")
    L, A = oracle.gemv_rows(w, k, x, threads=threads)
    o_am, o_nc = oracle.argmax_flags(L, A)
    w_d, x_d = to_dev(w), to_dev(x)
    del w

    log(f"max size n={n} k={k}: kq_gemv_rows m={m} and m=1")
    G = kq.gemv_rows(w_d, n, k, x_d)
    G1 = kq.gemv_rows(w_d, n, k, x_d[:1].contiguous())
    torch.cuda.synchronize()
    G, G1 = G.cpu().numpy(), G1.cpu().numpy()
    ratio = check_logits(G, L, A, what=f"max size {n}x{k}")
    log(f"max size n={n} k={k}: max |d|/tol = {ratio:.3g}")
    assert np.array_equal(G1[0], G[0]), "row 0 of the one-row call differs from the full call"

    log(f"max size n={n} k={k}: kq_verify_argmax_accept")
    drafts = [synthetic.forced_draft(o_am[:m - 1], (m - 1) // 2, n),
              synthetic.inject_mismatches(o_am[:m - 1], n, seed=seed + 2)]
    for i, d in enumerate(drafts):
        am, acc, lg = kq.verify(w_d, n, k, x_d, list(d), want_logits=(i == 0))
        torch.cuda.synchronize()
        am, acc = am.cpu().numpy(), acc.cpu().numpy()
        check_argmax(am, L, A, what=f"max size {n}x{k} trial {i}")
        check_accept(acc[0], acc[1], d, am, o_am, o_nc, what=f"max size {n}x{k} trial {i}")
        if lg is not None:
            assert np.array_equal(lg.cpu().numpy(), G), "verify logits differ from the product's"

    log(f"max size n={n} k={k}: tiled layout, staged product and one-phase chain")
    wt = kq.tile_weights(w_d, n, k)
    del w_d
    st = kq.stage_rows(x_d)
    sc = kq.new_scratch(n, k, DEV)
    T = kq.gemv_staged(wt, n, k, st, m, sc, layout=kq.LAYOUT_TILED16)
    out = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    chain = kq.chain_encode([([wt], n, k, st, [out])], m, layout=kq.LAYOUT_TILED16)
    kq.gemv_chain(chain)
    chain.status()
    torch.cuda.synchronize()
    assert np.array_equal(T.cpu().numpy(), G), "tiled weights give other logits than rows"
    C = out.cpu().numpy()
    if kq.launch_geometry(n, k)[:2] == (8, 1):  # the chain's own geometry
        assert np.array_equal(C, G), "chain logits differ from the single launch's"
    else:
        check_logits(C, L, A, what=f"max size chain {n}x{k}")
    del wt, st, sc, T, out, chain
    torch.cuda.empty_cache()


# The most weight bytes below 4 GiB for each row-group geometry: 128-row
# groups (8 one-tile waves; plain products on the specialised-wave kernel),
# 192 rows (12 waves; a ragged last tile) and 256 rows (8 two-tile waves,
# the LM head's instance).
MAX_WEIGHTS = [(32767, 232960, (8, 1)), (131071, 58112, (12, 1)), (131072, 58112, (8, 2))]


@pytest.mark.parametrize("n,k,geom", MAX_WEIGHTS)
def test_weights_just_under_4gib(kq, n, k, geom):
    wb = kq.tiled_bytes(n, k)
    assert LIMIT - 16 * 1024 * 1024 < wb < LIMIT and kq.tiled_bytes(n, k + 256) == 0
    assert kq.launch_geometry(n, k)[:2] == geom
    run_all(kq, n, k, 16, 700 + n % 97)


def test_staged_activations_just_under_4gib(kq):
    # k/256 staged blocks of 16,960 bytes: the largest k below 4 GiB, one
    # 128-row group whose 253,240 blocks every workgroup shares
    n, k = 17, 253240 * 256
    sb = kq.staged_bytes(k, 2)
    assert LIMIT - 16960 <= sb < LIMIT and kq.staged_bytes(k + 256, 2) == 0
    assert kq.launch_geometry(n, k) == (8, 1, 256, 253240)
    run_all(kq, n, k, 2, 900, threads=4)
