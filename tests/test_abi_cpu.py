"""CPU checks of the C ABI (no GPU): libkq.so loads, exports every function
include/kq.h declares, and every argument error is reported before any HIP
call (the fake device pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from quant_verify_gemv_amd import lib as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")

NULL, SHAPE, ALIGN, TOKEN, WS = 1, 2, 3, 4, 5
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = kq.load()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kq.EXPORTED)


def test_every_export_has_a_prototype():
    lib = kq.load()
    for n in kq.EXPORTED:
        fn = getattr(lib, n)
        if n != "kq_status_string":
            assert fn.argtypes is not None, f"{n} has no argtypes"
    assert lib.kq_group_scratch_bytes.restype is ctypes.c_size_t
    assert lib.kq_workspace_bytes.restype is ctypes.c_size_t


def test_status_strings():
    for code, name in kq.STATUS_NAMES.items():
        assert kq.status_string(code).startswith(name)
    assert kq.status_string(99) == "KQ_ERR_UNKNOWN"


def test_sizes_and_geometry():
    assert kq.workspace_bytes(512, 1000, 4) == 0       # k not a multiple of 256
    assert kq.workspace_bytes(512, 1024, 0) == 0
    assert kq.workspace_bytes(512, 1024, 65) == 0      # at most 64 rows
    assert kq.workspace_bytes(0, 1024, 1) == 0
    assert kq.staged_bytes(1024) == 4 * 16960
    assert kq.staged_bytes(6656) == 26 * 16960
    # more than 16 rows: one sixteen-row slice per 16 rows or part of them
    assert [kq.staged_bytes(1024, m) for m in (1, 16, 17, 32, 33, 48, 49, 64)] == \
        [4 * 16960 * s for s in (1, 1, 2, 2, 3, 3, 4, 4)]
    assert kq.staged_bytes(1024, 65) == 0 and kq.staged_bytes(1024, 0) == 0
    # the workspace grows with the slices of m: staged bytes and split-K partials
    ws = [kq.workspace_bytes(512, 1024, m) for m in (16, 32, 48, 64)]
    assert all(b - a >= 4 * 16960 for a, b in zip(ws, ws[1:]))
    for n, k in [(512, 1024), (6656, 6656), (6656, 33280), (131072, 6656), (17920, 6656), (6656, 17920), (1, 256),
                 (35840, 6656)]:
        assert kq.workspace_bytes(n, k, 1) == kq.workspace_bytes(n, k, 16) > 0
        assert kq.workspace_bytes(n, k, 64) > kq.workspace_bytes(n, k, 16)
        waves, tpw, nwg, units = kq.launch_geometry(n, k)
        assert waves in (4, 8, 12) and tpw in (1, 2)
        assert units == -(-n // (16 * waves * tpw)) * (k // 256)
        assert 1 <= nwg <= min(units, 768)
        a256 = -(-kq.staged_bytes(k, 64) // 256) * 256
        assert kq.workspace_bytes(n, k, 64) == a256 + kq.scratch_bytes(n, k)
    with pytest.raises(kq.KQError):
        kq.launch_geometry(16, 100)


def _call_gemv(w=FAKE, n=512, k=1024, x=FAKE, m=4, out=FAKE, ws=FAKE, wsb=None):
    lib = kq.load()
    if wsb is None:
        wsb = kq.workspace_bytes(n, k, m) or 1 << 30
    return lib.kq_gemv_rows(w, n, k, x, m, out, ws, wsb, None)


def _call_verify(w=FAKE, n=512, k=1024, x=FAKE, m=4, draft=(1, 2, 3), am=FAKE, acc=FAKE, lg=None,
                 ws=FAKE, wsb=None):
    lib = kq.load()
    if wsb is None:
        wsb = kq.workspace_bytes(n, k, m) or 1 << 30
    d = (ctypes.c_int32 * max(1, len(draft)))(*draft) if draft is not None else None
    return lib.kq_verify_argmax_accept(w, n, k, x, m, d, am, acc, lg, ws, wsb, None)


def test_gemv_argument_errors():
    assert _call_gemv(w=None) == NULL
    assert _call_gemv(x=None) == NULL
    assert _call_gemv(out=None) == NULL
    assert _call_gemv(ws=None) == NULL
    assert _call_gemv(m=0) == SHAPE
    assert _call_gemv(m=65) == SHAPE
    assert _call_gemv(k=1000) == SHAPE
    assert _call_gemv(k=0) == SHAPE
    assert _call_gemv(n=0) == SHAPE
    assert _call_gemv(n=1 << 31) == SHAPE
    assert _call_gemv(w=FAKE + 8) == ALIGN
    assert _call_gemv(x=FAKE + 4) == ALIGN
    assert _call_gemv(ws=FAKE + 16) == ALIGN
    assert _call_gemv(wsb=kq.workspace_bytes(512, 1024, 4) - 1) == WS


def test_four_gib_limits():
    # the weight matrix (rows rounded up to 16) must be smaller than 4 GiB
    assert 131072 * 227 * 144 < 1 << 32 <= 131072 * 228 * 144
    assert kq.workspace_bytes(131072, 227 * 256, 16) > 0
    assert kq.workspace_bytes(131072, 228 * 256, 16) == 0
    assert _call_gemv(n=131072, k=228 * 256, wsb=1 << 40) == SHAPE
    # n is rounded up to a whole 16-row tile
    q = 1864135
    assert 16 * q * 144 < 1 << 32 <= 16 * (q + 1) * 144
    assert kq.scratch_bytes(16 * q, 256) > 0
    assert kq.scratch_bytes(16 * q + 1, 256) == 0
    # the staged activations must be smaller than 4 GiB
    kb = (1 << 32) // 16960
    assert kb * 16960 < 1 << 32 <= (kb + 1) * 16960
    assert kq.scratch_bytes(1, kb * 256) > 0
    assert kq.scratch_bytes(1, (kb + 1) * 256) == 0


def test_verify_argument_errors():
    assert _call_verify(am=None) == NULL
    assert _call_verify(acc=None) == NULL
    assert _call_verify(draft=None) == NULL
    assert _call_verify(m=65, draft=tuple(range(64))) == SHAPE
    assert _call_verify(draft=(1, 2, 512)) == TOKEN
    assert _call_verify(draft=(-1, 2, 3)) == TOKEN
    assert _call_verify(wsb=100) == WS


def test_draft_block_argument_errors():
    lib = kq.load()
    n, k = 512, 1024

    def call(w=FAKE, x=FAKE, vl=7, props=FAKE, head=None, ws=FAKE, wsb=None):
        if wsb is None:
            wsb = kq.workspace_bytes(n, k, 16)
        return lib.kq_draft_block_argmax(w, n, k, x, vl, props, head, ws, wsb, None)

    # verify lengths other than 3, 7 and 15 are refused before any GPU work
    for vl in (-1, 0, 1, 2, 4, 5, 6, 8, 14, 16, 31):
        assert call(vl=vl) == SHAPE, vl
    assert call(w=None) == NULL
    assert call(x=None) == NULL
    assert call(props=None) == NULL
    assert call(ws=None) == NULL
    assert call(x=FAKE + 4) == ALIGN
    assert call(wsb=kq.workspace_bytes(n, k, 8) - 1) == WS
    sb = kq.scratch_bytes(n, k)
    st = lib.kq_draft_block_argmax_staged
    assert st(FAKE, 0, n, k, FAKE, 4, FAKE, None, FAKE, sb, None) == SHAPE
    assert st(FAKE, 7, n, k, FAKE, 3, FAKE, None, FAKE, sb, None) == SHAPE
    assert st(FAKE, 0, n, k, None, 3, FAKE, None, FAKE, sb, None) == NULL
    assert st(FAKE, 0, n, k, FAKE, 3, None, None, FAKE, sb, None) == NULL
    assert st(FAKE, 0, n, k, FAKE, 15, FAKE, None, FAKE, 256, None) == WS
    with pytest.raises(ValueError):
        kq.draft_block_argmax(None, n, k, None, 5)
    assert kq.DRAFT_VERIFY_LENGTHS == (3, 7, 15)


def test_stream_probe_argument_errors():
    lib = kq.load()
    sb = lib.kq_stream_probe_sink_bytes()
    assert sb > 0
    assert lib.kq_stream_probe(None, 1024, FAKE, sb, None) == NULL
    assert lib.kq_stream_probe(FAKE, 1024, None, sb, None) == NULL
    assert lib.kq_stream_probe(FAKE, 0, FAKE, sb, None) == SHAPE
    assert lib.kq_stream_probe(FAKE, 1000, FAKE, sb, None) == SHAPE
    assert lib.kq_stream_probe(FAKE + 8, 1024, FAKE, sb, None) == ALIGN
    assert lib.kq_stream_probe(FAKE, 1024, FAKE, sb - 4, None) == WS


def test_staged_argument_errors():
    lib = kq.load()
    assert lib.kq_stage_rows(None, 4, 1024, FAKE, 1 << 20, None) == NULL
    assert lib.kq_stage_rows(FAKE, 0, 1024, FAKE, 1 << 20, None) == SHAPE
    assert lib.kq_stage_rows(FAKE, 4, 1024, FAKE + 16, 1 << 20, None) == ALIGN
    assert lib.kq_stage_rows(FAKE, 4, 1024, FAKE, 100, None) == WS
    sb = kq.scratch_bytes(512, 1024)
    assert lib.kq_gemv_staged(FAKE, 0, 512, 1024, None, 4, FAKE, FAKE, sb, None) == NULL
    assert lib.kq_gemv_staged(FAKE, 0, 512, 1024, FAKE, 4, FAKE, FAKE, 256, None) == WS
    assert lib.kq_gemv_staged(FAKE, 7, 512, 1024, FAKE, 4, FAKE, FAKE, sb, None) == SHAPE
    assert lib.kq_gemv_staged(FAKE, -1, 512, 1024, FAKE, 4, FAKE, FAKE, sb, None) == SHAPE
    d = (ctypes.c_int32 * 3)(0, 1, 600)
    assert lib.kq_verify_staged(FAKE, 0, 512, 1024, FAKE, 4, d, FAKE, FAKE, None, FAKE, sb, None) == TOKEN
    assert lib.kq_verify_staged(FAKE, 1, 512, 1024, FAKE, 4, d, FAKE, FAKE, None, FAKE, sb, None) == TOKEN
    assert lib.kq_workspace_init(None, 256, None) == NULL
    assert lib.kq_workspace_init(FAKE + 4, 256, None) == ALIGN
    assert lib.kq_workspace_init(FAKE, 8, None) == WS


def test_grouped_argument_errors():
    lib = kq.load()
    n, k, m = 2000, 6656, 16
    sb = kq.group_scratch_bytes(n, k, 3)
    assert sb >= kq.scratch_bytes(n, k) > 0
    assert kq.group_scratch_bytes(n, k, 0) == 0 and kq.group_scratch_bytes(n, k, 9) == 0
    wp = (ctypes.c_void_p * 3)(FAKE, FAKE + 0x100000, FAKE + 0x200000)
    lp = (ctypes.c_void_p * 3)(FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000)
    call = lib.kq_gemv_staged_group
    for layout in (0, 1):
        assert call(wp, layout, 0, n, k, FAKE, m, lp, FAKE, sb, None) == SHAPE
        assert call(wp, layout, 9, n, k, FAKE, m, lp, FAKE, sb, None) == SHAPE
        assert call(wp, layout, 3, n, 100, FAKE, m, lp, FAKE, sb, None) == SHAPE
        assert call(wp, layout, 3, n, k, FAKE, m, lp, FAKE, 256, None) == WS
        assert call(None, layout, 3, n, k, FAKE, m, lp, FAKE, sb, None) == NULL
        bad = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
        assert call(bad, layout, 3, n, k, FAKE, m, lp, FAKE, sb, None) == NULL
        mis = (ctypes.c_void_p * 3)(FAKE, FAKE + 8, FAKE)
        assert call(mis, layout, 3, n, k, FAKE, m, lp, FAKE, sb, None) == ALIGN
    assert call(wp, 7, 3, n, k, FAKE, m, lp, FAKE, sb, None) == SHAPE


def test_tiling_sizes_and_argument_errors():
    lib = kq.load()
    assert kq.tiled_bytes(512, 1024) == 32 * 4 * 2304
    assert kq.tiled_bytes(17, 256) == 2 * 1 * 2304       # rows padded to 16
    assert kq.tiled_bytes(16, 100) == 0
    n, k = 1000, 2048
    nb = kq.tiled_bytes(n, k)
    rowmajor = n * (k // 256) * 144
    assert nb == 63 * 8 * 2304 and nb >= rowmajor
    out = FAKE + 0x40000000
    tw = lib.kq_tile_weights
    assert tw(None, n, k, out, nb, None) == NULL
    assert tw(FAKE, n, k, None, nb, None) == NULL
    assert tw(FAKE, n, 100, out, nb, None) == SHAPE
    assert tw(FAKE + 8, n, k, out, nb, None) == ALIGN
    assert tw(FAKE, n, k, out + 4, nb, None) == ALIGN
    assert tw(FAKE, n, k, out, nb - 1, None) == WS
    assert tw(FAKE, n, k, FAKE + 4096, nb, None) == SHAPE    # overlapping buffers


def test_q5k_q6k_tiling_sizes_and_argument_errors():
    lib = kq.load()
    L5, L6 = kq.LAYOUT_Q5K_TILED16, kq.LAYOUT_Q6K_TILED16
    assert kq.tiled_bytes(512, 1024, "q5k") == 32 * 4 * 16 * 176
    assert kq.tiled_bytes(17, 256, "q6k") == 2 * 1 * 16 * 210
    assert lib.kq_tiled_bytes_fmt(kq.LAYOUT_ROWS, 16, 256) == 0     # not a tiled layout
    assert lib.kq_tiled_bytes_fmt(9, 16, 256) == 0                  # unknown layout
    assert lib.kq_tiled_bytes_fmt(kq.LAYOUT_TILED16, 100, 512) == kq.tiled_bytes(100, 512)
    n, k = 1000, 2048
    out = FAKE + 0x40000000
    tf = lib.kq_tile_weights_fmt
    for lay in (L5, L6):
        nb = lib.kq_tiled_bytes_fmt(lay, n, k)
        assert tf(lay, None, n, k, out, nb, None) == NULL
        assert tf(lay, FAKE, n, k, None, nb, None) == NULL
        assert tf(lay, FAKE, n, 100, out, nb, None) == SHAPE
        assert tf(lay, FAKE, n, k, out + 4, nb, None) == ALIGN
        assert tf(lay, FAKE, n, k, out, nb - 1, None) == WS
        assert tf(lay, FAKE, n, k, FAKE + 4096, nb, None) == SHAPE  # overlapping buffers
    assert tf(L5, FAKE + 8, n, k, out, 1 << 30, None) == ALIGN       # Q5_K rows are 16-byte aligned
    assert tf(L6, FAKE + 1, n, k, out, 1 << 30, None) == ALIGN       # Q6_K rows: 2-byte aligned
    assert tf(kq.LAYOUT_ROWS, FAKE, n, k, out, 1 << 30, None) == SHAPE
    assert tf(6, FAKE, n, k, out, 1 << 30, None) == SHAPE
    # the staged calls take the Q5_K / Q6_K layouts (checked up to the launch)
    sb = kq.scratch_bytes(n, k)
    lp = (ctypes.c_void_p * 1)(FAKE)
    for lay in (L5, L6):
        assert lib.kq_gemv_staged(FAKE + 8, lay, n, k, FAKE, 16, FAKE, FAKE, sb, None) == ALIGN
        assert lib.kq_gemv_staged(FAKE, lay, n, k, FAKE, 16, FAKE, FAKE, 256, None) == WS
        assert lib.kq_gemv_staged(FAKE, lay, n, 100, FAKE, 16, FAKE, FAKE, sb, None) == SHAPE
    # scratch sized for any format: at least what each format's geometry needs
    assert kq.scratch_bytes(131072, 6656) > 0 and kq.group_scratch_bytes(2000, 6656, 3) > 0


def test_chain_refuses_q5k_q6k_layouts():
    for lay in (kq.LAYOUT_Q5K_TILED16, kq.LAYOUT_Q6K_TILED16):
        assert _encode([_phase()], layout=lay) == SHAPE


def _phase(count=2, n=512, k=1024, w=FAKE, logits=FAKE, staged=FAKE):
    ph = kq.ChainPhase()
    ph.count, ph.n, ph.k = count, n, k
    for j in range(min(count, kq.MAX_GROUP)):
        ph.w_q4k[j] = w
        ph.logits[j] = logits
    ph.staged = staged
    return ph


def _encode(phases, m=16, layout=kq.LAYOUT_ROWS, table_bytes=None, table=True, plan=True):
    lib = kq.load()
    n = len(phases)
    arr = (kq.ChainPhase * max(1, n))(*phases)
    tb = kq.chain_table_bytes(n) if table_bytes is None else table_bytes
    host = (ctypes.c_uint8 * max(1, tb))() if table else None
    pl = kq.ChainPlan()
    return lib.kq_chain_encode(arr, n, m, layout, host, tb, ctypes.byref(pl) if plan else None)


def test_chain_table_bytes():
    assert kq.chain_table_bytes(0) == 0
    assert kq.chain_table_bytes(65537) == 0
    one = kq.chain_table_bytes(1)
    assert one > 0 and kq.chain_table_bytes(208) == 208 * one


def test_chain_encode_argument_errors_before_any_hip_call():
    good = _phase()
    assert _encode([good], table=False) == NULL
    assert _encode([good], plan=False) == NULL
    assert _encode([good], m=0) == SHAPE
    assert _encode([good], m=17) == SHAPE
    assert _encode([good], layout=2) == SHAPE
    assert _encode([_phase(count=0)]) == SHAPE
    assert _encode([_phase(count=9)]) == SHAPE
    assert _encode([good, _phase(k=1000)]) == SHAPE          # k not a multiple of 256
    assert _encode([good, _phase(n=0)]) == SHAPE
    assert _encode([good, _phase(w=0)]) == NULL
    assert _encode([good, _phase(logits=0)]) == NULL
    assert _encode([good, _phase(staged=0)]) == NULL
    assert _encode([good, _phase(w=FAKE + 8)]) == ALIGN      # weights 16-byte aligned
    assert _encode([good, _phase(staged=FAKE + 16)]) == ALIGN  # staged 256-byte aligned
    assert _encode([good, good], table_bytes=kq.chain_table_bytes(2) - 1) == WS
    lib = kq.load()
    pl = kq.ChainPlan()
    assert lib.kq_chain_encode(None, 1, 16, 0, None, 0, ctypes.byref(pl)) == NULL
    arr = (kq.ChainPhase * 1)(good)
    host = (ctypes.c_uint8 * 1024)()
    assert lib.kq_chain_encode(arr, 0, 16, 0, host, 1024, ctypes.byref(pl)) == SHAPE


def test_gemv_chain_argument_errors_before_any_hip_call():
    lib = kq.load()
    pl = kq.ChainPlan()
    pl.n_phases, pl.m, pl.layout, pl.workgroups, pl.max_groups, pl.tiles_per_wave = 2, 16, 0, 256, 4, 1
    assert lib.kq_gemv_chain(None, ctypes.byref(pl), FAKE, 1 << 30, None) == NULL
    assert lib.kq_gemv_chain(FAKE, None, FAKE, 1 << 30, None) == NULL
    assert lib.kq_gemv_chain(FAKE, ctypes.byref(pl), None, 1 << 30, None) == NULL
    # a plan kq_chain_encode did not write (scratch_bytes inconsistent)
    assert lib.kq_gemv_chain(FAKE, ctypes.byref(pl), FAKE, 1 << 30, None) == SHAPE
    for field, bad in (("n_phases", 0), ("m", 0), ("m", 17), ("workgroups", 0), ("layout", 5), ("max_groups", 0),
                       ("tiles_per_wave", 3)):
        q = kq.ChainPlan.from_buffer_copy(pl)
        setattr(q, field, bad)
        assert lib.kq_gemv_chain(FAKE, ctypes.byref(q), FAKE, 1 << 30, None) == SHAPE, field
    assert lib.kq_gemv_chain(FAKE + 8, ctypes.byref(pl), FAKE, 1 << 30, None) == ALIGN
    assert lib.kq_gemv_chain(FAKE, ctypes.byref(pl), FAKE + 16, 1 << 30, None) == ALIGN


def test_chain_scratch_init_argument_errors_before_any_hip_call():
    lib = kq.load()
    pl = kq.ChainPlan()
    pl.n_phases, pl.m, pl.layout, pl.workgroups, pl.max_groups, pl.tiles_per_wave = 2, 16, 0, 256, 4, 1
    assert lib.kq_chain_scratch_init(None, FAKE, 1 << 30, None) == NULL
    assert lib.kq_chain_scratch_init(ctypes.byref(pl), None, 1 << 30, None) == NULL
    assert lib.kq_chain_scratch_init(ctypes.byref(pl), FAKE, 1 << 30, None) == SHAPE  # inconsistent scratch_bytes


def test_chain_status_argument_errors_before_any_hip_call():
    lib = kq.load()
    pl = kq.ChainPlan()
    pl.n_phases, pl.m, pl.layout, pl.workgroups, pl.max_groups, pl.tiles_per_wave = 2, 16, 0, 256, 4, 1
    assert lib.kq_chain_status(None, FAKE, 1 << 30, None) == NULL
    assert lib.kq_chain_status(ctypes.byref(pl), None, 1 << 30, None) == NULL
    assert lib.kq_chain_status(ctypes.byref(pl), FAKE, 1 << 30, None) == SHAPE  # inconsistent scratch_bytes
    q = kq.ChainPlan.from_buffer_copy(pl)
    q.m = 0
    assert lib.kq_chain_status(ctypes.byref(q), FAKE, 1 << 30, None) == SHAPE
    assert lib.kq_chain_status(ctypes.byref(pl), FAKE + 16, 1 << 30, None) == ALIGN


def test_noalloc_verify_argument_errors_before_any_hip_call():
    """The allocation-free verify refuses every bad argument with the code
    kq_verify_argmax_accept gives, and a shape whose workspace exceeds the
    library's fixed array with KQ_ERR_WORKSPACE, before any HIP call (there
    is no GPU here: a call that reached the device lookup would report
    KQ_ERR_LAUNCH)."""
    lib = kq.load()
    n, k = 512, 1024
    dr = (ctypes.c_int32 * 3)(1, 2, 3)

    def call(w=FAKE, n=n, k=k, x=FAKE, m=4, draft=dr, am=FAKE, acc=FAKE):
        return lib.kq_verify_argmax_accept_noalloc(w, n, k, x, m, draft, am, acc, None, None)
    assert call(w=None) == NULL and call(x=None) == NULL
    assert call(am=None) == NULL and call(acc=None) == NULL
    assert call(draft=None) == NULL
    assert call(k=1000) == SHAPE and call(m=0) == SHAPE and call(m=65) == SHAPE and call(n=0) == SHAPE
    assert call(w=FAKE + 8) == ALIGN and call(x=FAKE + 4) == ALIGN
    bad = (ctypes.c_int32 * 3)(1, n, 3)
    assert call(draft=bad) == TOKEN
    # 4,096 blocks per row: 69 MB of staged activations, over the fixed array
    big_k = 256 * 4096
    assert kq.workspace_bytes(n, big_k, 4) > 24 << 20
    assert call(k=big_k) == WS


def test_tree_verify_argument_errors_before_any_hip_call():
    lib = kq.load()
    n, k = 512, 1024
    sb = kq.scratch_bytes(n, k)

    def call(m=5, parent=(-1, 0, 0, 1, 2), token=(0, 1, 2, 3, 4), argmax=FAKE, acc=FAKE, path=None,
             layout=kq.LAYOUT_TILED16, scratch_bytes=sb):
        par = (ctypes.c_int32 * max(1, len(parent)))(*parent) if parent is not None else None
        tok = (ctypes.c_int32 * max(1, len(token)))(*token) if token is not None else None
        return lib.kq_verify_tree_staged(FAKE, layout, n, k, FAKE, m, par, tok, argmax, acc, path, None, FAKE,
                                         scratch_bytes, None)
    assert call(parent=None) == NULL and call(token=None) == NULL
    assert call(argmax=None) == NULL and call(acc=None) == NULL
    assert call(parent=(0, 0, 0, 1, 2)) == SHAPE          # the root has no parent
    assert call(parent=(-1, 0, 3, 1, 2)) == SHAPE         # a parent after its child
    assert call(parent=(-1, 0, 0, 1, -1)) == SHAPE
    assert call(token=(0, 1, 2, 3, n)) == TOKEN           # token outside [0, n)
    assert call(token=(0, 1, -2, 3, 4)) == TOKEN
    assert call(m=65, parent=(-1,) + tuple(range(64)), token=(0,) * 65) == SHAPE
    assert call(layout=7) == SHAPE
    assert call(scratch_bytes=256) == WS


def test_verify_staged_dev_argument_errors_before_any_hip_call():
    lib = kq.load()
    n, k, m = 512, 1024, 4
    sb = kq.scratch_bytes(n, k)
    v = lib.kq_verify_staged_dev
    assert v(FAKE, 1, n, k, FAKE, m, FAKE, None, FAKE, None, FAKE, sb, None) == NULL
    assert v(FAKE, 1, n, k, FAKE, m, FAKE, FAKE, None, None, FAKE, sb, None) == NULL
    assert v(FAKE, 1, n, k, FAKE, m, None, FAKE, FAKE, None, FAKE, sb, None) == NULL   # drafts needed for m > 1
    assert v(FAKE, 1, n, k, FAKE, m, FAKE + 2, FAKE, FAKE, None, FAKE, sb, None) == ALIGN
    assert v(FAKE, 1, n, k, FAKE, 65, FAKE, FAKE, FAKE, None, FAKE, sb, None) == SHAPE
    assert v(FAKE, 9, n, k, FAKE, m, FAKE, FAKE, FAKE, None, FAKE, sb, None) == SHAPE
    assert v(FAKE, 1, n, k, FAKE, m, FAKE, FAKE, FAKE, None, FAKE, 256, None) == WS


def test_gather_argument_errors():
    """kq_gather_rows checks its arguments before any HIP call; count = 0
    enqueues nothing."""
    lib = kq.load()
    p = ctypes.c_void_p(256)
    assert lib.kq_gather_rows(p, 0, 10, p, 0, p, None) == 2          # m < 1
    assert lib.kq_gather_rows(p, 4, 0, p, 1, p, None) == 2           # n < 1
    assert lib.kq_gather_rows(p, 4, 10, p, 5, p, None) == 2          # count > m
    assert lib.kq_gather_rows(p, 4, 10, p, -1, p, None) == 2         # count < 0
    assert lib.kq_gather_rows(None, 4, 10, p, 2, p, None) == 1
    assert lib.kq_gather_rows(p, 4, 10, None, 2, p, None) == 1
    assert lib.kq_gather_rows(p, 4, 10, p, 2, None, None) == 1
    assert lib.kq_gather_rows(ctypes.c_void_p(258), 4, 10, p, 2, p, None) == 3
    assert lib.kq_gather_rows(None, 4, 10, None, 0, None, None) == 0  # nothing to do
