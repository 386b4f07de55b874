"""GPU tests of the stochastic verify: the target probability rows
(kq_softmax_rows) against the oracle's fp64 softmax within the bound the fp32
arithmetic allows, the whole step at the LM-head size (verify logits ->
probability rows -> host decision) against the oracle's decision, also in
two steps from gathered p_i[d_i] and one copied row, and kq_gather_rows."""
import numpy as np
import pytest

import synthetic
from oracle.stochastic import softmax_rows as oracle_softmax
from oracle.stochastic import speculative_decide as oracle_decide
from tests.parity import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def check_probs(G, L, temperature, cap, what):
    """|p_gpu - p| <= p (8 * 2^-24 (max|z| + 1) + 1e-5) + 1e-37, z = l / T.

    Where the bound comes from: z = l / T is rounded once (relative 2^-24,
    a little more under the soft cap's tanh); exp(z - max) then carries an
    argument error below 4 max|z| 2^-24 plus about 2 ulp of expf; the
    chunk sums (16 terms per thread, a 256-wide tree) and the chunk combine
    add a relative error of a few 1e-6 at most, covered by the 1e-5 term;
    the final division one more rounding. The absolute 1e-37 admits the
    fp32 subnormal range, where relative precision is lost."""
    P = oracle_softmax(L, temperature, cap)
    zmax = np.abs(L.astype(np.float64)).max(axis=1, keepdims=True)
    if cap > 0:
        zmax = np.minimum(zmax, cap)
    zmax = zmax / temperature
    tol = P * (8 * 2.0 ** -24 * (zmax + 1) + 1e-5) + 1e-37
    err = np.abs(G.astype(np.float64) - P)
    bad = err > tol
    assert np.all(np.isfinite(G)), f"{what}: non-finite probabilities"
    assert not bad.any(), f"{what}: {int(bad.sum())} outside tolerance; first {np.argwhere(bad)[0]}"
    return float((err / tol).max())


@pytest.mark.parametrize("m,n", [(1, 1), (3, 7), (16, 4096), (5, 4097), (16, 50000)])
@pytest.mark.parametrize("temperature,cap", [(1.0, 0.0), (0.7, 30.0), (250.0, 0.0)])
def test_softmax_rows_vs_oracle(kq, m, n, temperature, cap):
    rng = np.random.default_rng(m * 1000 + n)
    L = (rng.normal(size=(m, n)) * (8.0 if temperature < 100 else 600.0)).astype(np.float32)
    Ld = torch.from_numpy(L).to(DEV)
    G = kq.softmax_rows(Ld, temperature, cap)
    G2 = kq.softmax_rows(Ld, temperature, cap)
    torch.cuda.synchronize()
    Gh = G.cpu().numpy()
    assert np.array_equal(Gh, G2.cpu().numpy()), "not deterministic"
    r = check_probs(Gh, L, temperature, cap, f"softmax m={m} n={n} T={temperature} cap={cap}")
    log(f"softmax m={m} n={n} T={temperature} cap={cap}: max err / tol = {r:.3g}")


def test_stochastic_verify_lm_head(kq):
    """The LM-head verify at full size (6,656 -> 131,072, 16 rows, tiled
    weights as the benchmark runs it): logits from the verify kernel, target
    rows from kq_softmax_rows at T = 300 (the synthetic logits spread over
    hundreds), draft rows from perturbed logits, proposals drawn from them.
    The library's decision equals the oracle's on the GPU's own rows bit for
    bit, and equals the oracle's on the oracle's fp64 rows except where a
    draw falls within the rows' tolerance of a decision boundary (counted)."""
    h = synthetic.LM_HEAD
    n, k, m = h["n"], h["k"], h["m"]
    kd = m - 1
    w = synthetic.q4k_matrix(n, k, h["seed"])
    x = synthetic.activations(m, k, h["seed"])
    wt = kq.tile_weights(torch.from_numpy(w).to(DEV), n, k)
    st = kq.stage_rows(torch.from_numpy(x).to(DEV))
    scratch = kq.new_scratch(n, k, DEV)
    am = torch.empty(m, dtype=torch.int32, device=DEV)
    acc = torch.empty(2, dtype=torch.int32, device=DEV)
    lg = torch.empty((m, n), dtype=torch.float32, device=DEV)
    kq.verify_staged(wt, n, k, st, m, [0] * kd, scratch, out=(am, acc, lg), layout=kq.LAYOUT_TILED16)
    T = 300.0
    P = kq.softmax_rows(lg, T)
    torch.cuda.synchronize()
    Lh, Ph = lg.cpu().numpy(), P.cpu().numpy()
    r = check_probs(Ph, Lh, T, 0.0, "LM-head rows")
    log(f"stochastic LM head: probability rows max err / tol = {r:.3g}")
    Pref = oracle_softmax(Lh, T).astype(np.float32)
    rng = np.random.default_rng(7)
    same_gpu = same_ref = boundary = 0
    accepted_hist = []
    orders = np.stack([np.argsort(-Ph[i], kind="stable") for i in range(m)]).astype(np.int32)
    for trial in range(24):
        noisy = Lh[:kd] + rng.normal(size=(kd, n)).astype(np.float32) * np.float32(40.0 + 20 * (trial % 4))
        q = oracle_softmax(noisy, T).astype(np.float32)
        qd = q.astype(np.float64)
        draft = [int(rng.choice(n, p=qd[i] / qd[i].sum())) for i in range(kd)]
        u = rng.random(m).astype(np.float32)
        got = kq.speculative_decide(draft, q, Ph, orders, u)
        assert got == oracle_decide(draft, q, Ph, orders, u), f"trial {trial}: library != oracle on the same rows"
        # the same decision from p_i[d_i] gathered on the device and one row copied
        p_at = kq.gather_rows(P[:kd], torch.tensor(draft, dtype=torch.int32, device=DEV)).cpu().numpy()
        assert np.array_equal(p_at, Ph[np.arange(kd), draft])
        j = kq.speculative_first_reject(p_at, q[np.arange(kd), draft], u[:kd])
        row = P[j].cpu().numpy()
        tok = (kq.speculative_resample(row, q[j], orders[j], u[j + 1]) if j < kd
               else kq.speculative_resample(row, None, orders[kd], u[kd]))
        assert (j, tok) == got, f"trial {trial}: two-step decision"
        same_gpu += 1
        want = oracle_decide(draft, q, Pref, orders, u)
        if got == want:
            same_ref += 1
        else:
            # only a draw within tolerance of a boundary may flip the decision
            i = min(got[0], want[0])
            ratio = Pref[i, draft[i]] / q[i, draft[i]] if i < kd else 1.0
            near = i < kd and abs(u[i] - min(ratio, 1.0)) < 1e-3
            assert near or got[0] == want[0], f"trial {trial}: decision differs away from any boundary"
            boundary += 1
        accepted_hist.append(got[0])
    log(f"stochastic LM head: {same_gpu} trials bitwise with the oracle on the GPU rows, {same_ref} equal "
        f"on the oracle's rows, {boundary} at a boundary; accepted lengths {sorted(accepted_hist)}")
    assert same_ref >= 20


def test_gather_rows(kq):
    """kq_gather_rows equals indexing on the host bit for bit; tokens
    outside the row give NaN; a count below m reads only the first rows."""
    rng = np.random.default_rng(3)
    m, n = 16, 70001
    R = rng.random((m, n)).astype(np.float32)
    tok = rng.integers(0, n, m).astype(np.int32)
    tok[3], tok[9] = -1, n
    Rd = torch.from_numpy(R).to(DEV)
    got = kq.gather_rows(Rd, torch.from_numpy(tok).to(DEV)).cpu().numpy()
    ok = (tok >= 0) & (tok < n)
    assert np.array_equal(got[ok], R[np.arange(m)[ok], tok[ok]])
    assert np.all(np.isnan(got[~ok]))
    few = kq.gather_rows(Rd, torch.from_numpy(tok[:5].copy()).to(DEV)).cpu().numpy()
    assert few.shape == (5,) and np.array_equal(few[[0, 1, 2, 4]], R[[0, 1, 2, 4], tok[[0, 1, 2, 4]]])
