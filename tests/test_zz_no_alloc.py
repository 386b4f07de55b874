"""GPU test of kq_verify_argmax_accept_noalloc, the allocation-free verify
(its workspace is the library's fixed device array): called through the C
ABI twice in a row, the LM-head shape and then a smaller one, each compared
bit for bit with kq_verify_argmax_accept on a workspace of its own (same
kernels, same geometry): logits, argmax and the accept decision; the smaller
call's logits also against the oracle; calls of two slices and one slice in
turn; and the call captured in a HIP graph."""
import ctypes

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


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def verify_both(kq, w, n, k, x, draft):
    """(noalloc outputs, workspace-call outputs), each (argmax, accept, logits)."""
    lib = kq.lib.load()
    m = x.shape[0]
    dr = (ctypes.c_int32 * max(1, m - 1))(*[int(t) for t in draft])
    outs = []
    for noalloc in (True, False):
        am = torch.full((m,), -7, dtype=torch.int32, device=DEV)
        acc = torch.full((2,), -7, dtype=torch.int32, device=DEV)
        lg = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
        if noalloc:
            rc = lib.kq_verify_argmax_accept_noalloc(p(w), n, k, p(x), m, dr, p(am), p(acc), p(lg), None)
        else:
            ws = kq.lib.alloc_workspace(kq.workspace_bytes(n, k, m), DEV)
            rc = lib.kq_verify_argmax_accept(p(w), n, k, p(x), m, dr, p(am), p(acc), p(lg), p(ws), ws.numel(),
                                             None)
        assert rc == 0, kq.status_string(rc)
        torch.cuda.synchronize()
        outs.append((am.cpu().numpy(), acc.cpu().numpy(), lg.cpu().numpy()))
    return outs


def test_noalloc_verify_matches_workspace_call_twice(kq):
    cases = [(synthetic.VOCAB, synthetic.HIDDEN, 16, 3), (1000, 2304, 5, 91)]
    for n, k, m, seed in cases:
        log(f"noalloc: n={n} k={k} m={m}")
        w = synthetic.q4k_matrix(n, k, seed)
        x = synthetic.activations(m, k, seed + 1)
        draft = [int(t) for t in np.random.default_rng(seed).integers(0, n, m - 1)]
        wd = torch.from_numpy(w).to(DEV)
        xd = torch.from_numpy(x).to(DEV)
        (am_a, acc_a, lg_a), (am_b, acc_b, lg_b) = verify_both(kq, wd, n, k, xd, draft)
        assert np.array_equal(am_a, am_b), "argmax differs from the workspace call"
        assert np.array_equal(acc_a, acc_b), "accept differs from the workspace call"
        assert np.array_equal(lg_a.view(np.uint32), lg_b.view(np.uint32)), "logits differ from the workspace call"
        if n <= 4096:
            L, A = oracle.gemv_rows(w, k, x)
            check_logits(lg_a, L, A, what=f"noalloc n={n} k={k} m={m}")


def test_noalloc_verify_more_rows_then_fewer(kq):
    """Calls of different slice counts on the one device array: a 24-row
    call (two slices) puts its staged rows, and so its control words and
    partials, at other offsets than the 8-row call after it. Each equals the
    workspace call bit for bit, and its logits the oracle."""
    n, k = 2000, 2304
    w = synthetic.q4k_matrix(n, k, 95)
    wd = torch.from_numpy(w).to(DEV)
    for m in (24, 8, 24):
        log(f"noalloc: n={n} k={k} m={m}")
        x = synthetic.activations(m, k, 96 + m)
        draft = [int(t) for t in np.random.default_rng(97 + m).integers(0, n, m - 1)]
        (am_a, acc_a, lg_a), (am_b, acc_b, lg_b) = verify_both(kq, wd, n, k, torch.from_numpy(x).to(DEV), draft)
        assert np.array_equal(am_a, am_b) and np.array_equal(acc_a, acc_b), f"m={m}: argmax or accept"
        assert np.array_equal(lg_a.view(np.uint32), lg_b.view(np.uint32)), f"m={m}: logits"
        L, A = oracle.gemv_rows(w, k, x)
        check_logits(lg_a, L, A, what=f"noalloc m={m}")


def test_noalloc_verify_replays_from_a_graph(kq):
    """The caller it is for: the call captured in a HIP graph (nothing is
    allocated during capture; the draft tokens travel in the kernel
    arguments). Every replay gives the eager call's argmax, accept and
    logits bit for bit, also after an eager call of another shape has used
    the same device array in between."""
    lib = kq.lib.load()
    n, k, m = 3000, 2304, 8
    w = torch.from_numpy(synthetic.q4k_matrix(n, k, 77)).to(DEV)
    x = torch.from_numpy(synthetic.activations(m, k, 78)).to(DEV)
    draft = [int(t) for t in np.random.default_rng(79).integers(0, n, m - 1)]
    dr = (ctypes.c_int32 * (m - 1))(*draft)
    am = torch.full((m,), -7, dtype=torch.int32, device=DEV)
    acc = torch.full((2,), -7, dtype=torch.int32, device=DEV)
    lg = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)

    def call():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.kq_verify_argmax_accept_noalloc(p(w), n, k, p(x), m, dr, p(am), p(acc), p(lg), s)
        assert rc == 0, kq.status_string(rc)

    call()
    torch.cuda.synchronize()
    ref = (am.cpu().numpy(), acc.cpu().numpy(), lg.cpu().numpy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    other_w = torch.from_numpy(synthetic.q4k_matrix(700, 1024, 80)).to(DEV)
    other_x = torch.from_numpy(synthetic.activations(5, 1024, 81)).to(DEV)
    for r in range(3):
        am.fill_(-7)
        acc.fill_(-7)
        lg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = (am.cpu().numpy(), acc.cpu().numpy(), lg.cpu().numpy())
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), f"replay {r}: argmax or accept"
        assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32)), f"replay {r}: logits"
        verify_both(kq, other_w, 700, 1024, other_x, [1, 2, 3, 4])  # another shape on the same array
