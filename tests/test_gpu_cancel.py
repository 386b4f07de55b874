"""GPU parity where the scale term and the min term of a Q4_K weight cancel.

The kernel contracts the exact fp16 operands sc_j q_k with the activations and
the exact 6-bit mins m_j with the sub-block sums of the activations, then forms
d * C - dmin * C_m per block in fp32: its rounding error is proportional to
B = sum_k (|d sc_j q_k| + |dmin m_j|) |x_k| (oracle.term_mass), not to the
tolerance mass A = sum_k |w_k x_k|. The two agree for the configured
workloads (weights biased positive, B/A about 1.3); real quantizers centre
the weights on zero (dmin m_j near 7.5 d sc_j here, B/A about 4); a weight with
d sc_j q_k = dmin m_j contributes to B but not to A.

* Centred weights (synthetic.q4k_matrix_centred) at the LM-head and square
  shapes: every logit within the declared tolerance 1e-4 * A, argmax with
  flags, accept.
* Rows built from blocks whose every weight cancels exactly (w = 0, d and
  dmin nonzero), alone and mixed with random blocks: every logit within the
  kernel's stated worst-case bound 2^-24 (544 + k/128) B (include/kq.h);
  rows with A > 0 are also held to 1e-4 * A wherever that is the larger."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_accept, check_argmax, check_logits, log
from tests.q4k_pack import f16_bits, pack_block

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def kernel_bound(k, B):
    """The worst-case error bound include/kq.h states for the kernel,
    2^-24 (544 + k/128) B, with 1/256 of it added for the absolute floor of
    activations below 2^-12 of their block's largest magnitude (at most
    2^-34 of that magnitude per activation: for N(0, 1) rows, whose block
    maxima are about 3, far less than that)."""
    return 2.0 ** -24 * (544 + k / 128) * B * (1 + 2.0 ** -8)


def test_centred_weights_lm_head_verify(kq):
    n, k, m = synthetic.VOCAB, synthetic.HIDDEN, 16
    w = synthetic.q4k_matrix_centred(n, k, 71)
    x = synthetic.activations(m, k, 72)
    log("cancel: oracle of the centred LM head")
    L, A = oracle.gemv_rows(w, k, x)
    draft = synthetic.inject_mismatches(oracle.argmax_flags(L, A)[0][:m - 1], n, 73)
    wd = torch.from_numpy(w).to(DEV)
    am, acc, lg = kq.verify(wd, n, k, torch.from_numpy(x).to(DEV), list(draft), want_logits=True)
    G = lg.cpu().numpy()
    ratio = check_logits(G, L, A, what="centred LM head")
    o_am, o_nc, flagged = check_argmax(am.cpu().numpy(), L, A, what="centred LM head")
    a = acc.cpu().numpy()
    check_accept(a[0], a[1], draft, am.cpu().numpy(), o_am, o_nc, what="centred LM head")
    B = oracle.term_mass(w, k, x, rows=np.arange(0, n, 97))
    log(f"cancel: centred LM head max |err|/(1e-4 A) = {ratio:.2e}, flagged rows {flagged}, "
        f"mean B/A on sampled rows {float(np.mean(B / A[:, ::97])):.2f}")


@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_centred_weights_square_every_m(kq, layout):
    n = k = synthetic.HIDDEN
    w = synthetic.q4k_matrix_centred(n, k, 74)
    x = synthetic.activations(16, k, 75)
    L, A = oracle.gemv_rows(w, k, x)
    wd = torch.from_numpy(w).to(DEV)
    lay = kq.LAYOUT_ROWS
    if layout == "tiled":
        wd = kq.tile_weights(wd, n, k)
        lay = kq.LAYOUT_TILED16
    scratch = kq.new_scratch(n, k, DEV)
    for m in (1, 2, 4, 8, 16):
        st = kq.stage_rows(torch.from_numpy(x[:m]).to(DEV))
        G = kq.gemv_staged(wd, n, k, st, m, scratch, layout=lay).cpu().numpy()
        ratio = check_logits(G, L[:m], A[:m], what=f"centred square {layout} m={m}")
        log(f"cancel: centred square {layout} m={m} max |err|/(1e-4 A) = {ratio:.2e}")


def test_exactly_cancelling_blocks(kq):
    """300 rows x 9 blocks, M = 16. Rows r % 3 == 0: every block cancels
    (d = dmin drawn per block, sc = 4, q = 15, m = 60, so every weight is
    d (60 - 60) = 0: L = A = 0); rows r % 3 == 1: cancelling and random
    blocks alternate; rows r % 3 == 2: random blocks only."""
    n, k, m = 300, 2304, 16
    rng = np.random.default_rng(76)
    rand = synthetic.q4k_matrix(n, k, 77).reshape(n, k // 256, 144)
    w = rand.copy()
    for r in range(n):
        for b in range(k // 256):
            if r % 3 == 0 or (r % 3 == 1 and b % 2 == 0):
                d = f16_bits(float(rng.uniform(0.001, 0.05)))
                w[r, b] = np.frombuffer(pack_block(d, d, [4] * 8, [60] * 8, [15] * 256), dtype=np.uint8)
    w = w.reshape(n, -1)
    x = synthetic.activations(m, k, 78)
    L, A = oracle.gemv_rows(w, k, x)
    B = oracle.term_mass(w, k, x)
    assert np.all(L[:, ::3] == 0.0) and np.all(A[:, ::3] == 0.0)
    G = kq.gemv_rows(torch.from_numpy(w).to(DEV), n, k, torch.from_numpy(x).to(DEV)).cpu().numpy()
    err = np.abs(G.astype(np.float64) - L)
    bound = kernel_bound(k, B)
    assert np.all(np.isfinite(G))
    worst = float(np.max(err / bound))
    assert np.all(err <= bound), f"{int((err > bound).sum())} logits outside the kernel's stated bound"
    # where the declared tolerance is the larger, it holds too
    tol = oracle.REL_TOL * A
    looser = tol >= bound
    assert np.all(err[looser] <= tol[looser])
    zero_rows = float(np.max(np.abs(G[:, ::3])))
    log(f"cancel: exact cancellation max |err|/bound = {worst:.2e}, largest |logit| on w = 0 rows {zero_rows:.3e}")
