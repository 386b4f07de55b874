"""GPU parity of the benchmarked step itself: the synthetic 52-layer stack
(364 Q4_K matrices as 208 dependent phases, q,k,v | o | gate,up | down per
layer, tiled weights, one chain launch) followed by the LM-head verify, built
and run by bench.py's own Stack class, at M = 16 and M = 1.

Every one of the 364 stack matrices is checked against the oracle on sampled
rows that include the row-group edges of every launch geometry (0, 1, 127,
128, 191, 192, 255, 256 and n - 1), plus seeded random rows. The LM head's
oracle logits are computed in full, so its argmax (with flags) and the accept
decision are checked as in the single-launch verify tests. A graph replay of
the step is compared bitwise with the eager step (the bench times replays)."""
import numpy as np
import pytest

import oracle
import synthetic
from tests.parity import check_accept, check_argmax, check_logits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EDGES = (0, 1, 127, 128, 191, 192, 255, 256)


@pytest.fixture(scope="module")
def kq():
    import quant_verify_gemv_amd as kq
    kq.load()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return kq


def sample_rows(n, rng, extra=24):
    r = [e for e in EDGES if e < n] + [n - 1] + [int(v) for v in rng.integers(0, n, extra)]
    return np.unique(np.array(r, dtype=np.int64))


def test_benchmarked_stack_step_vs_oracle(kq, capsys):
    import bench

    def say(msg):
        with capsys.disabled():
            print(msg, flush=True)

    xs = {k: synthetic.activations(16, k, synthetic.stack_activation_seed(k))
          for k in (synthetic.HIDDEN, synthetic.FFN)}
    rng = np.random.default_rng(2024)
    ref = {}

    def on_matrix(i, g, w_host):
        if g.n == synthetic.VOCAB:  # the LM head: every row, for the argmax
            L, A = oracle.gemv_rows(w_host, g.k, xs[g.k])
            ref["head"] = (L, A)
        else:
            rows = sample_rows(g.n, rng)
            L, A = oracle.gemv_rows(w_host, g.k, xs[g.k], rows=rows)
            ref[i] = (rows, L, A)
        if i % 52 == 0:
            say(f"stack parity: oracle rows of matrix {i}")

    stack = bench.Stack(kq, torch, DEV, synthetic.LAYERS, kq.LAYOUT_TILED16, "chain", on_matrix=on_matrix)
    assert len(stack.mats) == 364 and len(stack.groups) == 208
    Lh, Ah = ref["head"]
    worst = 0.0
    for m in (16, 1):
        say(f"stack parity: eager step at m={m}")
        for o in stack.out:
            o.fill_(float("nan"))
        stack.step(m)
        torch.cuda.synchronize()
        assert stack.chain(m).error_word() == 0, "a chain barrier timed out"
        for i, g in enumerate(stack.mats):
            rows, L, A = ref[i]
            got = stack.out[i][:m].cpu().numpy()[:, rows]
            worst = max(worst, check_logits(got, L[:m], A[:m], what=f"stack matrix {i} ({g.n}x{g.k}) m={m}"))
        am = stack.am[:m].cpu().numpy()
        acc = stack.acc.cpu().numpy()
        o_am, o_nc, flagged = check_argmax(am, Lh[:m], Ah[:m], what=f"stack LM head m={m}")
        check_accept(acc[0], acc[1], stack.draft[:m - 1], am, o_am, o_nc, what=f"stack LM head m={m}")
        say(f"stack parity: m={m} all 364 matrices and the LM head checked "
            f"(worst |err|/tol so far {worst:.2e}, flagged head rows {flagged})")
        # the bench times graph replays: one replay must reproduce the eager step
        eager = stack.snapshot(m)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            stack.step(m)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            stack.step(m)
        g.replay()
        assert bench.same(stack.snapshot(m), eager), f"graph replay differs from the eager step at m={m}"
        del g
