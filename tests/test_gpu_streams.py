"""Concurrent calls on two HIP streams, each with its own workspace (GPU).

The single-launch kernels combine split row groups by last arrival (an
atomic count, never a wait on another workgroup), so two launches may share
the CUs in any proportion. Two unrelated problems are enqueued alternately
on two default-priority streams with no synchronisation between them, eight
rounds each, every round writing fresh output buffers:

* stream 1: kq_gemv_rows on the 6,656 x 6,656 square matrix, M = 16
  (workspace 1);
* stream 2: kq_verify_argmax_accept on a 32,768 x 6,656 head, M = 8 with 7
  draft tokens (workspace 2), and kq_gemv_staged on the tiled square matrix
  with a scratch of its own.

Every output of every round must equal, bit for bit, the same call made
alone on one stream beforehand (the kernels are deterministic), and those
reference outputs are checked against the oracle on sampled rows."""
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


def test_two_streams_with_separate_workspaces(kq):
    nA = kA = synthetic.HIDDEN
    nB, kB, mB = 32768, synthetic.HIDDEN, 8
    wA_h = synthetic.q4k_matrix(nA, kA, 301)
    wB_h = synthetic.q4k_matrix(nB, kB, 302)
    xA_h = synthetic.activations(16, kA, 303)
    xB_h = synthetic.activations(mB, kB, 304)
    wA, wB = torch.from_numpy(wA_h).to(DEV), torch.from_numpy(wB_h).to(DEV)
    xA, xB = torch.from_numpy(xA_h).to(DEV), torch.from_numpy(xB_h).to(DEV)
    wA_t = kq.tile_weights(wA, nA, kA)
    stA = kq.stage_rows(xA)
    draft = list(range(100, 100 + mB - 1))

    ws1 = kq.lib.alloc_workspace(kq.workspace_bytes(nA, kA, 16), DEV)
    ws2 = kq.lib.alloc_workspace(kq.workspace_bytes(nB, kB, mB), DEV)
    sc2 = kq.new_scratch(nA, kA, DEV)

    # references: each call alone
    refA = kq.gemv_rows(wA, nA, kA, xA, workspace=ws1)
    amB, accB, lgB = kq.verify(wB, nB, kB, xB, draft, want_logits=True, workspace=ws2)
    refS = kq.gemv_staged(wA_t, nA, kA, stA, 16, sc2, layout=kq.LAYOUT_TILED16)
    torch.cuda.synchronize()
    refA, refS = refA.clone(), refS.clone()
    amB, accB, lgB = amB.clone(), accB.clone(), lgB.clone()

    rows = np.unique(np.concatenate([[0, 1, 127, 128, nA - 1], np.random.default_rng(305).integers(0, nA, 40)]))
    L, A = oracle.gemv_rows(wA_h, kA, xA_h, rows=rows)
    check_logits(refA.cpu().numpy()[:, rows], L, A, what="square (stream reference)")
    check_logits(refS.cpu().numpy()[:, rows], L, A, what="square staged (stream reference)")
    LB, AB = oracle.gemv_rows(wB_h, kB, xB_h)
    check_logits(lgB.cpu().numpy(), LB, AB, what="head verify (stream reference)")
    check_argmax(amB.cpu().numpy(), LB, AB, what="head verify (stream reference)")

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(8):
        oA = torch.full((16, nA), float("nan"), device=DEV)
        oS = torch.full((16, nA), float("nan"), device=DEV)
        oam = torch.full((mB,), -1, dtype=torch.int32, device=DEV)
        oacc = torch.full((2,), -1, dtype=torch.int32, device=DEV)
        olg = torch.full((mB, nB), float("nan"), device=DEV)
        torch.cuda.synchronize()  # the fills are done before either stream starts
        kq.gemv_rows(wA, nA, kA, xA, logits=oA, workspace=ws1, stream=s1)
        kq.verify(wB, nB, kB, xB, draft, want_logits=True, workspace=ws2, stream=s2, out=(oam, oacc, olg))
        kq.gemv_staged(wA_t, nA, kA, stA, 16, sc2, logits=oS, stream=s2, layout=kq.LAYOUT_TILED16)
        kq.gemv_rows(wA, nA, kA, xA, logits=oA, workspace=ws1, stream=s1)  # again, the same result
        outs.append((oA, oS, oam, oacc, olg))
    torch.cuda.synchronize()
    for rep, (oA, oS, oam, oacc, olg) in enumerate(outs):
        assert torch.equal(oA, refA), f"round {rep}: stream-1 logits differ from the call alone"
        assert torch.equal(oS, refS), f"round {rep}: stream-2 staged logits differ from the call alone"
        assert torch.equal(oam, amB) and torch.equal(oacc, accB), f"round {rep}: stream-2 argmax / accept differ"
        assert torch.equal(olg, lgB), f"round {rep}: stream-2 verify logits differ"
    log("streams: 8 concurrent rounds on two streams equal the calls made alone")


def test_two_streams_with_default_workspaces(kq):
    """Calls that leave the workspace out on two streams at once: the
    binding keeps one default workspace per device and stream, so the two
    streams' calls never share a buffer. Eight rounds of kq_gemv_rows on
    stream 1 and kq_verify_argmax_accept on stream 2, enqueued alternately
    with no ordering between the streams, each equal bit for bit to the
    same call made alone on its own workspace."""
    nA = kA = synthetic.HIDDEN
    nB, kB, mB = 32768, synthetic.HIDDEN, 8
    wA = torch.from_numpy(synthetic.q4k_matrix(nA, kA, 311)).to(DEV)
    wB = torch.from_numpy(synthetic.q4k_matrix(nB, kB, 312)).to(DEV)
    xA = torch.from_numpy(synthetic.activations(16, kA, 313)).to(DEV)
    xB = torch.from_numpy(synthetic.activations(mB, kB, 314)).to(DEV)
    draft = list(range(200, 200 + mB - 1))
    refA = kq.gemv_rows(wA, nA, kA, xA, workspace=kq.lib.alloc_workspace(kq.workspace_bytes(nA, kA, 16), DEV))
    amB, accB, lgB = kq.verify(wB, nB, kB, xB, draft, want_logits=True,
                               workspace=kq.lib.alloc_workspace(kq.workspace_bytes(nB, kB, mB), DEV))
    torch.cuda.synchronize()
    refA, amB, accB, lgB = refA.clone(), amB.clone(), accB.clone(), lgB.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(8):
        oA = torch.full((16, nA), float("nan"), device=DEV)
        oam = torch.full((mB,), -1, dtype=torch.int32, device=DEV)
        oacc = torch.full((2,), -1, dtype=torch.int32, device=DEV)
        olg = torch.full((mB, nB), float("nan"), device=DEV)
        torch.cuda.synchronize()  # the fills are done before either stream starts
        kq.gemv_rows(wA, nA, kA, xA, logits=oA, stream=s1)
        kq.verify(wB, nB, kB, xB, draft, want_logits=True, stream=s2, out=(oam, oacc, olg))
        outs.append((oA, oam, oacc, olg))
    torch.cuda.synchronize()
    for rep, (oA, oam, oacc, olg) in enumerate(outs):
        assert torch.equal(oA, refA), f"round {rep}: stream-1 logits differ from the call alone"
        assert torch.equal(oam, amB) and torch.equal(oacc, accB), f"round {rep}: stream-2 argmax / accept differ"
        assert torch.equal(olg, lgB), f"round {rep}: stream-2 verify logits differ"
    log("streams: default workspaces, 8 concurrent rounds on two streams equal the calls made alone")


def test_four_host_threads_each_with_its_own_stream(kq):
    """Host reentrancy: four Python threads enter the library at once (ctypes
    releases the interpreter lock during each call), each enqueueing twelve
    rounds of kq_gemv_rows and kq_verify_argmax_accept on a stream and a
    workspace of its own, for problems of different shapes, with no ordering
    between the threads. Every output equals its call made alone, bit for
    bit; those references match the oracle on sampled rows."""
    import threading

    shapes = [(synthetic.HIDDEN, synthetic.HIDDEN, 16), (2048, 9216, 4), (30000, 2304, 8), (513, 3328, 1)]
    probs = []
    for i, (n, k, m) in enumerate(shapes):
        w_h = synthetic.q4k_matrix(n, k, 400 + i)
        x_h = synthetic.activations(m, k, 410 + i)
        w, x = torch.from_numpy(w_h).to(DEV), torch.from_numpy(x_h).to(DEV)
        ws = kq.lib.alloc_workspace(kq.workspace_bytes(n, k, m), DEV)
        draft = [int(t) for t in np.random.default_rng(420 + i).integers(0, n, m - 1)]
        lg = kq.gemv_rows(w, n, k, x, workspace=ws)
        am, acc, vl = kq.verify(w, n, k, x, draft, want_logits=True, workspace=ws)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(430 + i).integers(0, n, 24)]))
        L, A = oracle.gemv_rows(w_h, k, x_h, rows=rows)
        check_logits(lg.cpu().numpy()[:, rows], L, A, what=f"thread problem {i} (reference)")
        assert torch.equal(vl, lg), f"problem {i}: verify logits differ from the product's"
        probs.append(dict(n=n, k=k, m=m, w=w, x=x, ws=ws, draft=draft, ref=(lg.clone(), am.clone(), acc.clone())))

    errors = []
    start = threading.Barrier(len(probs))

    def worker(i):
        try:
            p = probs[i]
            n, k, m = p["n"], p["k"], p["m"]
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(12):
                    lg = torch.full((m, n), float("nan"), device=DEV)
                    kq.gemv_rows(p["w"], n, k, p["x"], logits=lg, workspace=p["ws"], stream=s)
                    am, acc, _ = kq.verify(p["w"], n, k, p["x"], p["draft"], workspace=p["ws"], stream=s)
                    outs.append((lg, am, acc))
                s.synchronize()
                ref_lg, ref_am, ref_acc = p["ref"]
                for r, (lg, am, acc) in enumerate(outs):
                    if not (torch.equal(lg, ref_lg) and torch.equal(am, ref_am) and torch.equal(acc, ref_acc)):
                        errors.append(f"thread {i} round {r}: differs from the call made alone")
        except Exception as e:  # reported below, in the test's own thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    log("threads: 4 host threads x 12 rounds equal the calls made alone")
