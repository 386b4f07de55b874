"""Thin ctypes binding over libkq.so (the C ABI in include/kq.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the verify path runs in the HIP kernels. There is no
fallback: if libkq.so is missing or the device is not a HIP GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkq.so")

KQ_OK = 0
STATUS_NAMES = {0: "KQ_OK", 1: "KQ_ERR_NULL", 2: "KQ_ERR_SHAPE", 3: "KQ_ERR_ALIGN",
                4: "KQ_ERR_TOKEN", 5: "KQ_ERR_WORKSPACE", 6: "KQ_ERR_LAUNCH"}

EXPORTED = ("kq_status_string", "kq_workspace_bytes", "kq_staged_bytes", "kq_scratch_bytes",
            "kq_workspace_init", "kq_gemv_rows", "kq_verify_argmax_accept", "kq_stage_rows",
            "kq_gemv_staged", "kq_verify_staged", "kq_launch_geometry", "kq_group_scratch_bytes",
            "kq_gemv_staged_group", "kq_tiled_bytes", "kq_tile_weights", "kq_draft_block_argmax",
            "kq_draft_block_argmax_staged", "kq_stream_probe", "kq_stream_probe_sink_bytes",
            "kq_chain_table_bytes", "kq_chain_encode", "kq_gemv_chain", "kq_chain_scratch_init",
            "kq_softmax_workspace_bytes", "kq_softmax_rows", "kq_speculative_decide",
            "kq_tiled_bytes_fmt", "kq_tile_weights_fmt", "kq_staged_bytes_rows", "kq_verify_tree_staged",
            "kq_verify_staged_dev", "kq_gather_rows", "kq_speculative_first_reject", "kq_speculative_resample",
            "kq_chain_status", "kq_verify_argmax_accept_noalloc", "kq_mt19937_seed", "kq_mt19937_u32",
            "kq_mt19937_uniform_f32", "kq_speculative_decide_mt")

LAYOUT_ROWS = 0      # llama.cpp row-major blocks
LAYOUT_TILED16 = 1   # kq_tile_weights output
LAYOUT_Q5K_TILED16 = 2  # kq_tile_weights_fmt output for a Q5_K matrix
LAYOUT_Q6K_TILED16 = 3  # kq_tile_weights_fmt output for a Q6_K matrix
# weight format -> (tiled layout, bytes per 256-weight block in llama.cpp rows)
FORMATS = {"q4k": (LAYOUT_TILED16, 144), "q5k": (LAYOUT_Q5K_TILED16, 176), "q6k": (LAYOUT_Q6K_TILED16, 210)}

MAX_GROUP = 8
CHAIN_BARRIER_OFFSET = 128  # byte offset of the chain's barrier arrival count in its scratch
CHAIN_ERROR_OFFSET = 256    # byte offset of the chain's barrier time-out word in its scratch


class ChainPhase(ctypes.Structure):
    """kq_chain_phase (include/kq.h)."""
    _fields_ = [("count", ctypes.c_int), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("w_q4k", ctypes.c_void_p * MAX_GROUP), ("logits", ctypes.c_void_p * MAX_GROUP),
                ("staged", ctypes.c_void_p)]


class ChainPlan(ctypes.Structure):
    """kq_chain_plan (include/kq.h)."""
    _fields_ = [("n_phases", ctypes.c_int32), ("m", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("workgroups", ctypes.c_int32), ("max_groups", ctypes.c_int32), ("tiles_per_wave", ctypes.c_int32),
                ("table_bytes", ctypes.c_uint64), ("scratch_bytes", ctypes.c_uint64)]


class MT19937State(ctypes.Structure):
    """kq_mt19937 (include/kq.h): 624 state words and the next index."""
    _fields_ = [("mt", ctypes.c_uint32 * 624), ("index", ctypes.c_uint32)]


_lib = None


class KQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libkq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m quant_verify_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.kq_status_string.argtypes = [I32]
    lib.kq_status_string.restype = ctypes.c_char_p
    lib.kq_workspace_bytes.argtypes = [I64, I64, I32]
    lib.kq_workspace_bytes.restype = SZ
    lib.kq_staged_bytes.argtypes = [I64]
    lib.kq_staged_bytes.restype = SZ
    lib.kq_scratch_bytes.argtypes = [I64, I64]
    lib.kq_scratch_bytes.restype = SZ
    lib.kq_workspace_init.argtypes = [P, SZ, P]
    lib.kq_gemv_rows.argtypes = [P, I64, I64, P, I32, P, P, SZ, P]
    lib.kq_verify_argmax_accept.argtypes = [P, I64, I64, P, I32, P, P, P, P, P, SZ, P]
    lib.kq_stage_rows.argtypes = [P, I32, I64, P, SZ, P]
    lib.kq_gemv_staged.argtypes = [P, I32, I64, I64, P, I32, P, P, SZ, P]
    lib.kq_verify_staged.argtypes = [P, I32, I64, I64, P, I32, P, P, P, P, P, SZ, P]
    lib.kq_launch_geometry.argtypes = [I64, I64, P, P, P, P]  # int*, int*, int*, int64_t*
    lib.kq_draft_block_argmax.argtypes = [P, I64, I64, P, I32, P, P, P, SZ, P]
    lib.kq_stream_probe.argtypes = [P, SZ, P, SZ, P]
    lib.kq_stream_probe_sink_bytes.argtypes = []
    lib.kq_stream_probe_sink_bytes.restype = SZ
    lib.kq_draft_block_argmax_staged.argtypes = [P, I32, I64, I64, P, I32, P, P, P, SZ, P]
    lib.kq_group_scratch_bytes.argtypes = [I64, I64, I32]
    lib.kq_group_scratch_bytes.restype = SZ
    lib.kq_gemv_staged_group.argtypes = [P, I32, I32, I64, I64, P, I32, P, P, SZ, P]
    lib.kq_tiled_bytes.argtypes = [I64, I64]
    lib.kq_tiled_bytes.restype = SZ
    lib.kq_tile_weights.argtypes = [P, I64, I64, P, SZ, P]
    lib.kq_chain_table_bytes.argtypes = [I32]
    lib.kq_chain_table_bytes.restype = SZ
    lib.kq_chain_encode.argtypes = [ctypes.POINTER(ChainPhase), I32, I32, I32, P, SZ, ctypes.POINTER(ChainPlan)]
    lib.kq_gemv_chain.argtypes = [P, ctypes.POINTER(ChainPlan), P, SZ, P]
    lib.kq_chain_scratch_init.argtypes = [ctypes.POINTER(ChainPlan), P, SZ, P]
    lib.kq_chain_status.argtypes = [ctypes.POINTER(ChainPlan), P, SZ, P]
    lib.kq_verify_argmax_accept_noalloc.argtypes = [P, I64, I64, P, I32, P, P, P, P, P]
    lib.kq_softmax_workspace_bytes.argtypes = [I32, I64]
    lib.kq_softmax_workspace_bytes.restype = SZ
    F = ctypes.c_float
    lib.kq_softmax_rows.argtypes = [P, I32, I64, F, F, P, P, SZ, P]
    lib.kq_speculative_decide.argtypes = [I32, P, I64, P, P, P, P, P, P]
    lib.kq_gather_rows.argtypes = [P, I32, I64, P, I32, P, P]
    lib.kq_speculative_first_reject.argtypes = [I32, P, P, P, P]
    lib.kq_speculative_resample.argtypes = [I64, P, P, P, F, P]
    MTP = ctypes.POINTER(MT19937State)
    lib.kq_mt19937_seed.argtypes = [MTP, ctypes.c_uint32]
    lib.kq_mt19937_u32.argtypes = [MTP, P, I64]
    lib.kq_mt19937_uniform_f32.argtypes = [MTP, P, I64]
    lib.kq_speculative_decide_mt.argtypes = [I32, P, I64, P, P, P, MTP, P, P]
    lib.kq_verify_staged_dev.argtypes = [P, I32, I64, I64, P, I32, P, P, P, P, P, SZ, P]
    lib.kq_staged_bytes_rows.argtypes = [I64, I32]
    lib.kq_staged_bytes_rows.restype = SZ
    lib.kq_verify_tree_staged.argtypes = [P, I32, I64, I64, P, I32, P, P, P, P, P, P, P, SZ, P]
    lib.kq_tiled_bytes_fmt.argtypes = [I32, I64, I64]
    lib.kq_tiled_bytes_fmt.restype = SZ
    lib.kq_tile_weights_fmt.argtypes = [I32, P, I64, I64, P, SZ, P]
    for name in ("kq_workspace_init", "kq_gemv_rows", "kq_verify_argmax_accept", "kq_stage_rows",
                 "kq_gemv_staged", "kq_verify_staged", "kq_launch_geometry", "kq_gemv_staged_group",
                 "kq_tile_weights", "kq_draft_block_argmax", "kq_draft_block_argmax_staged",
                 "kq_stream_probe", "kq_chain_encode", "kq_gemv_chain", "kq_chain_scratch_init",
                 "kq_softmax_rows", "kq_speculative_decide", "kq_tile_weights_fmt", "kq_verify_tree_staged",
                 "kq_verify_staged_dev", "kq_gather_rows", "kq_speculative_first_reject",
                 "kq_speculative_resample", "kq_chain_status", "kq_verify_argmax_accept_noalloc",
                 "kq_mt19937_seed", "kq_mt19937_u32", "kq_mt19937_uniform_f32", "kq_speculative_decide_mt"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kq_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != KQ_OK:
        raise KQError(status, where)


def workspace_bytes(n: int, k: int, m: int) -> int:
    return int(load().kq_workspace_bytes(n, k, m))


def staged_bytes(k: int, m: int = 16) -> int:
    return int(load().kq_staged_bytes_rows(k, m))


def scratch_bytes(n: int, k: int) -> int:
    return int(load().kq_scratch_bytes(n, k))


def group_scratch_bytes(n: int, k: int, count: int) -> int:
    return int(load().kq_group_scratch_bytes(n, k, count))


def tiled_bytes(n: int, k: int, fmt: str = "q4k") -> int:
    return int(load().kq_tiled_bytes_fmt(FORMATS[fmt][0], n, k))


def launch_geometry(n: int, k: int) -> Tuple[int, int, int, int]:
    """(waves per workgroup, 16-row tiles per wave, persistent workgroups,
    units) the library uses for an n x k matrix; a unit is one row group of
    16 * waves * tiles rows times one 256-column block."""
    v = [ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int64(0)]
    _check(load().kq_launch_geometry(n, k, *[ctypes.byref(x) for x in v]), "kq_launch_geometry")
    return tuple(x.value for x in v)


# ----------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _dev_ptr(t, name: str, dtype=None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return int(t.data_ptr())


def alloc_workspace(nbytes: int, device):
    """A zeroed, 256-byte aligned device buffer of at least nbytes bytes."""
    torch = _torch()
    buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


class Workspace:
    """Default device workspaces, one per device and stream (grows as
    needed). Calls on different streams get different buffers, so calls that
    leave `workspace` out may overlap on two streams; calls on one stream are
    ordered and share its buffer. Each buffer is recorded as used by its
    stream, so the allocator does not hand a replaced buffer's memory to
    other work before that stream's pending calls are done, and the stream
    waits for the new buffer's zero fill."""

    def __init__(self):
        self._bufs = {}

    def get(self, nbytes: int, device, stream=None):
        torch = _torch()
        s = torch.cuda.current_stream(device) if stream is None else stream
        key = (str(device), int(s.cuda_stream))
        b = self._bufs.get(key)
        if b is None or b.numel() < nbytes:
            b = alloc_workspace(nbytes, device)  # zero-filled on the current stream
            s.wait_stream(torch.cuda.current_stream(device))
            b.record_stream(s)
            self._bufs[key] = b
        return b


_WS = Workspace()


def gemv_rows(w, n: int, k: int, x, logits=None, workspace=None, stream=None):
    """logits[m][n] = sum_k W[n][k] x[m][k] for a Q4_K matrix w (uint8 device
    tensor of n*(k/256)*144 bytes) and fp32 rows x [m, k]."""
    torch = _torch()
    if x.dim() == 1:
        x = x.unsqueeze(0)
    m = int(x.shape[0])
    if logits is None:
        logits = torch.empty((m, n), dtype=torch.float32, device=x.device)
    need = workspace_bytes(n, k, m)
    ws = workspace if workspace is not None else _WS.get(need, x.device, stream)
    _check(load().kq_gemv_rows(_dev_ptr(w, "w", torch.uint8), n, k, _dev_ptr(x, "x", torch.float32), m,
                               _dev_ptr(logits, "logits", torch.float32), _dev_ptr(ws, "workspace"),
                               ws.numel(), _stream_handle(stream)), "kq_gemv_rows")
    return logits


def verify(w, n: int, k: int, x, draft: Sequence[int], want_logits: bool = False,
           workspace=None, stream=None, out=None):
    """The verify step. Returns (argmax int32[m] device, accept int32[2]
    device = {accepted, next_token}, logits or None)."""
    torch = _torch()
    m = int(x.shape[0])
    dr = (ctypes.c_int32 * max(1, m - 1))(*[int(t) for t in draft])
    if len(draft) != m - 1:
        raise ValueError(f"need m-1 = {m - 1} draft tokens, got {len(draft)}")
    if out is None:
        am = torch.empty(m, dtype=torch.int32, device=x.device)
        acc = torch.empty(2, dtype=torch.int32, device=x.device)
        lg = torch.empty((m, n), dtype=torch.float32, device=x.device) if want_logits else None
    else:
        am, acc, lg = out
    need = workspace_bytes(n, k, m)
    ws = workspace if workspace is not None else _WS.get(need, x.device, stream)
    _check(load().kq_verify_argmax_accept(
        _dev_ptr(w, "w", torch.uint8), n, k, _dev_ptr(x, "x", torch.float32), m, dr,
        _dev_ptr(am, "argmax", torch.int32), _dev_ptr(acc, "accept", torch.int32),
        _dev_ptr(lg, "logits", torch.float32) if lg is not None else None,
        _dev_ptr(ws, "workspace"), ws.numel(), _stream_handle(stream)), "kq_verify_argmax_accept")
    return am, acc, lg


def stream_probe(buf, sink=None, stream=None):
    """Read every byte of the device tensor `buf` once (measurement helper).
    Returns the sink tensor (a checksum per workgroup)."""
    torch = _torch()
    lib = load()
    if sink is None:
        sink = torch.empty(lib.kq_stream_probe_sink_bytes() // 4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib.kq_stream_probe(_dev_ptr(buf, "buf"), nbytes, _dev_ptr(sink, "sink", torch.int32),
                               sink.numel() * 4, _stream_handle(stream)), "kq_stream_probe")
    return sink


DRAFT_VERIFY_LENGTHS = (3, 7, 15)


def draft_block_argmax(w, n: int, k: int, x, verify_length: int, want_head: bool = False,
                       workspace=None, stream=None, out=None):
    """The draft block's proposals: argmax of rows 1..verify_length of x
    (fp32 [>= verify_length + 1][k]) against the LM head w. Returns
    (proposals int32[verify_length] device, head int32[1] device or None)."""
    torch = _torch()
    if verify_length not in DRAFT_VERIFY_LENGTHS:
        raise ValueError(f"verify_length must be 3, 7 or 15, got {verify_length}")
    if int(x.shape[0]) < verify_length + 1:
        raise ValueError(f"x needs {verify_length + 1} rows, has {int(x.shape[0])}")
    if out is None:
        props = torch.empty(verify_length, dtype=torch.int32, device=x.device)
        head = torch.empty(1, dtype=torch.int32, device=x.device) if want_head else None
    else:
        props, head = out
    need = workspace_bytes(n, k, verify_length + 1)
    ws = workspace if workspace is not None else _WS.get(need, x.device, stream)
    _check(load().kq_draft_block_argmax(
        _dev_ptr(w, "w", torch.uint8), n, k, _dev_ptr(x, "x", torch.float32), verify_length,
        _dev_ptr(props, "proposals", torch.int32), _dev_ptr(head, "head", torch.int32) if head is not None else None,
        _dev_ptr(ws, "workspace"), ws.numel(), _stream_handle(stream)), "kq_draft_block_argmax")
    return props, head


def stage_rows(x, staged=None, stream=None):
    torch = _torch()
    m, k = int(x.shape[0]), int(x.shape[1])
    if staged is None:
        staged = alloc_workspace(staged_bytes(k, m), x.device)
    _check(load().kq_stage_rows(_dev_ptr(x, "x", torch.float32), m, k, _dev_ptr(staged, "staged"),
                                staged.numel(), _stream_handle(stream)), "kq_stage_rows")
    return staged


def new_scratch(n: int, k: int, device):
    """Zeroed scratch for the *_staged calls."""
    return alloc_workspace(scratch_bytes(n, k), device)


def tile_weights(w, n: int, k: int, out=None, stream=None, fmt: str = "q4k"):
    """The tiled copy (uint8 device tensor) of a matrix given as llama.cpp
    rows of format `fmt` ("q4k": KQ_LAYOUT_TILED16, "q5k", "q6k"); pass
    layout=FORMATS[fmt][0] to the staged calls."""
    torch = _torch()
    layout = FORMATS[fmt][0]
    nb = tiled_bytes(n, k, fmt)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=w.device)
    _check(load().kq_tile_weights_fmt(layout, _dev_ptr(w, "w", torch.uint8), n, k,
                                      _dev_ptr(out, "out", torch.uint8), out.numel(), _stream_handle(stream)),
           "kq_tile_weights_fmt")
    return out


def gemv_staged(w, n: int, k: int, staged, m: int, scratch, logits=None, stream=None, layout=LAYOUT_ROWS):
    torch = _torch()
    if logits is None:
        logits = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check(load().kq_gemv_staged(_dev_ptr(w, "w", torch.uint8), layout, n, k, _dev_ptr(staged, "staged"), m,
                                 _dev_ptr(logits, "logits", torch.float32), _dev_ptr(scratch, "scratch"),
                                 scratch.numel(), _stream_handle(stream)), "kq_gemv_staged")
    return logits


def new_group_scratch(n: int, k: int, count: int, device):
    """Zeroed scratch for kq_gemv_staged_group."""
    return alloc_workspace(group_scratch_bytes(n, k, count), device)


def gemv_staged_group(ws, n: int, k: int, staged, m: int, scratch, logits=None, stream=None,
                      layout=LAYOUT_ROWS):
    """One launch for several same-shape matrices sharing staged rows."""
    torch = _torch()
    count = len(ws)
    if logits is None:
        logits = [torch.empty((m, n), dtype=torch.float32, device=ws[0].device) for _ in range(count)]
    wp = (ctypes.c_void_p * count)(*[_dev_ptr(w, "w", torch.uint8) for w in ws])
    lp = (ctypes.c_void_p * count)(*[_dev_ptr(l, "logits", torch.float32) for l in logits])
    _check(load().kq_gemv_staged_group(wp, layout, count, n, k, _dev_ptr(staged, "staged"), m, lp,
                                       _dev_ptr(scratch, "scratch"), scratch.numel(),
                                       _stream_handle(stream)), "kq_gemv_staged_group")
    return logits


def draft_block_argmax_staged(w, n: int, k: int, staged, verify_length: int, scratch, want_head=False,
                              stream=None, out=None, layout=LAYOUT_ROWS):
    torch = _torch()
    if verify_length not in DRAFT_VERIFY_LENGTHS:
        raise ValueError(f"verify_length must be 3, 7 or 15, got {verify_length}")
    dev = staged.device
    if out is None:
        props = torch.empty(verify_length, dtype=torch.int32, device=dev)
        head = torch.empty(1, dtype=torch.int32, device=dev) if want_head else None
    else:
        props, head = out
    _check(load().kq_draft_block_argmax_staged(
        _dev_ptr(w, "w", torch.uint8), layout, n, k, _dev_ptr(staged, "staged"), verify_length,
        _dev_ptr(props, "proposals", torch.int32), _dev_ptr(head, "head", torch.int32) if head is not None else None,
        _dev_ptr(scratch, "scratch"), scratch.numel(), _stream_handle(stream)), "kq_draft_block_argmax_staged")
    return props, head


def verify_staged(w, n: int, k: int, staged, m: int, draft, scratch, want_logits=False,
                  stream=None, out=None, layout=LAYOUT_ROWS):
    """The verify step on staged activations. `draft` is a sequence of m-1
    host tokens (kq_verify_staged), or an int32 device tensor of m-1 tokens
    (kq_verify_staged_dev: no host round trip, no host range check)."""
    torch = _torch()
    on_device = hasattr(draft, "is_cuda") and draft.is_cuda
    if len(draft) != m - 1:
        raise ValueError(f"need m-1 = {m - 1} draft tokens, got {len(draft)}")
    if out is None:
        am = torch.empty(m, dtype=torch.int32, device=w.device)
        acc = torch.empty(2, dtype=torch.int32, device=w.device)
        lg = torch.empty((m, n), dtype=torch.float32, device=w.device) if want_logits else None
    else:
        am, acc, lg = out
    common = (_dev_ptr(am, "argmax", torch.int32), _dev_ptr(acc, "accept", torch.int32),
              _dev_ptr(lg, "logits", torch.float32) if lg is not None else None,
              _dev_ptr(scratch, "scratch"), scratch.numel(), _stream_handle(stream))
    if on_device:
        dp = _dev_ptr(draft, "draft", torch.int32) if m > 1 else None
        _check(load().kq_verify_staged_dev(_dev_ptr(w, "w", torch.uint8), layout, n, k, _dev_ptr(staged, "staged"),
                                           m, dp, *common), "kq_verify_staged_dev")
    else:
        dr = (ctypes.c_int32 * max(1, m - 1))(*[int(t) for t in draft])
        _check(load().kq_verify_staged(_dev_ptr(w, "w", torch.uint8), layout, n, k, _dev_ptr(staged, "staged"), m,
                                       dr, *common), "kq_verify_staged")
    return am, acc, lg


def verify_tree_staged(w, n: int, k: int, staged, parent: Sequence[int], token: Sequence[int], scratch,
                       want_logits=False, want_path=True, stream=None, out=None, layout=LAYOUT_ROWS):
    """Token-tree verify of m = len(parent) nodes (kq_verify_tree_staged):
    returns (argmax[m], accept[2] = {accepted, next_token}, path[m] or None,
    logits [m, n] or None), device int32 / fp32 tensors."""
    torch = _torch()
    m = len(parent)
    if len(token) != m:
        raise ValueError("parent and token need one entry per node")
    par = (ctypes.c_int32 * max(1, m))(*[int(v) for v in parent])
    tok = (ctypes.c_int32 * max(1, m))(*[int(v) for v in token])
    dev = w.device
    if out is None:
        am = torch.empty(m, dtype=torch.int32, device=dev)
        acc = torch.empty(2, dtype=torch.int32, device=dev)
        path = torch.full((m,), -1, dtype=torch.int32, device=dev) if want_path else None
        lg = torch.empty((m, n), dtype=torch.float32, device=dev) if want_logits else None
    else:
        am, acc, path, lg = out
    _check(load().kq_verify_tree_staged(
        _dev_ptr(w, "w", torch.uint8), layout, n, k, _dev_ptr(staged, "staged"), m, par, tok,
        _dev_ptr(am, "argmax", torch.int32), _dev_ptr(acc, "accept", torch.int32),
        _dev_ptr(path, "path", torch.int32) if path is not None else None,
        _dev_ptr(lg, "logits", torch.float32) if lg is not None else None,
        _dev_ptr(scratch, "scratch"), scratch.numel(), _stream_handle(stream)), "kq_verify_tree_staged")
    return am, acc, path, lg


# ------------------------------------------------------------------- chains

class Chain:
    """An encoded chain (kq_chain_encode): the device copy of its phase
    table, its plan, its scratch (zeroed once) and the tensors it refers to
    (kept alive with it)."""

    def __init__(self, table, plan, scratch, refs):
        self.table, self.plan, self.scratch, self._refs = table, plan, scratch, refs

    @property
    def workgroups(self) -> int:
        return int(self.plan.workgroups)

    def init_scratch(self, stream=None):
        """kq_chain_scratch_init on this chain's scratch (current stream)."""
        _check(load().kq_chain_scratch_init(ctypes.byref(self.plan), _dev_ptr(self.scratch, "scratch"),
                                            self.scratch.numel(), _stream_handle(stream)), "kq_chain_scratch_init")

    def error_word(self) -> int:
        """The barrier time-out word (synchronises with the device)."""
        off = CHAIN_ERROR_OFFSET
        return int(self.scratch[off:off + 4].view(_torch().int32).item())

    def status(self, stream=None):
        """kq_chain_status: waits for the stream, raises KQError
        (KQ_ERR_LAUNCH) when a wait of an earlier launch on this chain's
        scratch gave up (its logits are incomplete)."""
        _check(load().kq_chain_status(ctypes.byref(self.plan), _dev_ptr(self.scratch, "scratch"),
                                      self.scratch.numel(), _stream_handle(stream)), "kq_chain_status")


def chain_table_bytes(n_phases: int) -> int:
    return int(load().kq_chain_table_bytes(n_phases))


def chain_encode(phases, m: int, layout=LAYOUT_ROWS, device=None) -> Chain:
    """Encode a chain of dependent grouped products. `phases` is a sequence
    of (ws, n, k, staged, logits): ws a list of 1..8 uint8 device weight
    tensors of n x k (in `layout`), staged the kq_stage_rows block for k,
    logits a list of fp32 device tensors [>= m][n] (one per weight). The
    table is copied to the device once here."""
    torch = _torch()
    n_ph = len(phases)
    arr = (ChainPhase * max(1, n_ph))()
    refs = []
    for i, (ws, n, k, staged, logits) in enumerate(phases):
        if len(ws) != len(logits):
            raise ValueError(f"phase {i}: {len(ws)} weights but {len(logits)} logit buffers")
        if not 1 <= len(ws) <= MAX_GROUP:
            raise ValueError(f"phase {i}: 1..{MAX_GROUP} matrices per phase, got {len(ws)}")
        arr[i].count = len(ws)
        arr[i].n = int(n)
        arr[i].k = int(k)
        for j, (w, lg) in enumerate(zip(ws, logits)):
            arr[i].w_q4k[j] = _dev_ptr(w, "w", torch.uint8)
            arr[i].logits[j] = _dev_ptr(lg, "logits", torch.float32)
        arr[i].staged = _dev_ptr(staged, "staged")
        refs.extend(list(ws) + list(logits) + [staged])
    nbytes = max(1, chain_table_bytes(n_ph))
    host = (ctypes.c_uint8 * nbytes)()
    plan = ChainPlan()
    _check(load().kq_chain_encode(arr, n_ph, int(m), int(layout), host, nbytes, ctypes.byref(plan)),
           "kq_chain_encode")
    dev = device if device is not None else refs[0].device
    table = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(dev)
    scratch = alloc_workspace(int(plan.scratch_bytes), dev)
    chain = Chain(table, plan, scratch, refs)
    chain.init_scratch()
    return chain


def gemv_chain(chain: Chain, stream=None):
    """Run an encoded chain on the current stream (one launch)."""
    _check(load().kq_gemv_chain(_dev_ptr(chain.table, "table"), ctypes.byref(chain.plan),
                                _dev_ptr(chain.scratch, "scratch"), chain.scratch.numel(),
                                _stream_handle(stream)), "kq_gemv_chain")


# -------------------------------------------------------- stochastic verify

def softmax_workspace_bytes(m: int, n: int) -> int:
    return int(load().kq_softmax_workspace_bytes(m, n))


def softmax_rows(logits, temperature: float = 1.0, soft_cap: float = 0.0, probs=None, workspace=None,
                 stream=None):
    """Target probability rows (device fp32 [m, n]) from device logits [m, n]."""
    torch = _torch()
    m, n = int(logits.shape[0]), int(logits.shape[1])
    if probs is None:
        probs = torch.empty_like(logits)
    need = softmax_workspace_bytes(m, n)
    ws = workspace if workspace is not None else _WS.get(max(need, 256), logits.device, stream)
    _check(load().kq_softmax_rows(_dev_ptr(logits, "logits", torch.float32), m, n, float(temperature),
                                  float(soft_cap), _dev_ptr(probs, "probs", torch.float32), _dev_ptr(ws, "workspace"),
                                  ws.numel(), _stream_handle(stream)), "kq_softmax_rows")
    return probs


def speculative_decide(draft, draft_rows, target_rows, orders, uniforms):
    """The accept / resample decision on host arrays (numpy): draft [k],
    draft_rows fp32 [k, n], target_rows fp32 [k + 1, n], orders int32
    [k + 1, n], uniforms fp32 [k + 1]. Returns (accepted, next_token)."""
    import numpy as np
    k = len(draft)
    tr = np.ascontiguousarray(target_rows, dtype=np.float32)
    n = int(tr.shape[1])
    dr = np.ascontiguousarray(draft_rows, dtype=np.float32) if k else np.zeros((1, n), np.float32)
    od = np.ascontiguousarray(orders, dtype=np.int32)
    un = np.ascontiguousarray(uniforms, dtype=np.float32)
    dt = np.ascontiguousarray(draft, dtype=np.int32) if k else np.zeros(1, np.int32)
    if tr.shape[0] != k + 1 or od.shape != (k + 1, n) or un.shape != (k + 1,) or (k and dr.shape != (k, n)):
        raise ValueError("geometry: need k draft rows, k + 1 target rows, orders and uniforms")
    acc, nxt = ctypes.c_int32(0), ctypes.c_int32(0)
    vp = ctypes.c_void_p
    _check(load().kq_speculative_decide(k, vp(dt.ctypes.data), n, vp(dr.ctypes.data), vp(tr.ctypes.data),
                                        vp(od.ctypes.data), vp(un.ctypes.data), ctypes.byref(acc),
                                        ctypes.byref(nxt)), "kq_speculative_decide")
    return int(acc.value), int(nxt.value)


class MT19937:
    """The library's pinned draw stream (kq_mt19937_*): a host-owned state
    that the calls below advance. copy() snapshots it."""

    def __init__(self, seed: int = 5489):
        self.state = MT19937State()
        _check(load().kq_mt19937_seed(ctypes.byref(self.state), int(seed) & 0xFFFFFFFF), "kq_mt19937_seed")

    def copy(self) -> "MT19937":
        c = MT19937.__new__(MT19937)
        c.state = MT19937State()
        ctypes.memmove(ctypes.byref(c.state), ctypes.byref(self.state), ctypes.sizeof(MT19937State))
        return c

    def u32(self, count: int):
        import numpy as np
        out = np.zeros(max(int(count), 1), dtype=np.uint32)
        _check(load().kq_mt19937_u32(ctypes.byref(self.state), ctypes.c_void_p(out.ctypes.data), int(count)),
               "kq_mt19937_u32")
        return out[:int(count)]

    def uniform_f32(self, count: int):
        import numpy as np
        out = np.zeros(max(int(count), 1), dtype=np.float32)
        _check(load().kq_mt19937_uniform_f32(ctypes.byref(self.state), ctypes.c_void_p(out.ctypes.data),
                                             int(count)), "kq_mt19937_uniform_f32")
        return out[:int(count)]


def speculative_decide_mt(draft, draft_rows, target_rows, orders, rng: MT19937):
    """kq_speculative_decide_mt: the decision with its draws taken from rng
    (advanced by the draws consumed). Returns (accepted, next_token)."""
    import numpy as np
    k = len(draft)
    tr = np.ascontiguousarray(target_rows, dtype=np.float32)
    n = int(tr.shape[1])
    dr = np.ascontiguousarray(draft_rows, dtype=np.float32) if k else np.zeros((1, n), np.float32)
    od = np.ascontiguousarray(orders, dtype=np.int32)
    dt = np.ascontiguousarray(draft, dtype=np.int32) if k else np.zeros(1, np.int32)
    if tr.shape[0] != k + 1 or od.shape != (k + 1, n) or (k and dr.shape != (k, n)):
        raise ValueError("geometry: need k draft rows, k + 1 target rows and orders")
    acc, nxt = ctypes.c_int32(0), ctypes.c_int32(0)
    vp = ctypes.c_void_p
    _check(load().kq_speculative_decide_mt(k, vp(dt.ctypes.data), n, vp(dr.ctypes.data), vp(tr.ctypes.data),
                                           vp(od.ctypes.data), ctypes.byref(rng.state), ctypes.byref(acc),
                                           ctypes.byref(nxt)), "kq_speculative_decide_mt")
    return int(acc.value), int(nxt.value)


def gather_rows(rows, tokens, out=None, stream=None):
    """out[i] = rows[i, tokens[i]] on the device (kq_gather_rows): rows fp32
    [m, n], tokens int32 [count <= m] (device tensors). NaN for a token
    outside [0, n)."""
    torch = _torch()
    m, n = int(rows.shape[0]), int(rows.shape[1])
    count = int(tokens.numel())
    if out is None:
        out = torch.empty(max(count, 1), dtype=torch.float32, device=rows.device)
    if count:
        _check(load().kq_gather_rows(_dev_ptr(rows, "rows", torch.float32), m, n,
                                     _dev_ptr(tokens, "tokens", torch.int32), count,
                                     _dev_ptr(out, "out", torch.float32), _stream_handle(stream)), "kq_gather_rows")
    return out[:count]


def speculative_first_reject(p_at, q_at, uniforms):
    """The first rejected position (host arrays): p_at, q_at fp32 [k] =
    p_i[d_i], q_i[d_i]; uniforms fp32 [>= k]. Returns k when all accept."""
    import numpy as np
    pa = np.ascontiguousarray(p_at, dtype=np.float32)
    qa = np.ascontiguousarray(q_at, dtype=np.float32)
    un = np.ascontiguousarray(uniforms, dtype=np.float32)
    k = int(pa.shape[0])
    if qa.shape != (k,) or un.shape[0] < k:
        raise ValueError("need k values of p, of q and k draws")
    pos = ctypes.c_int32(0)
    vp = ctypes.c_void_p
    _check(load().kq_speculative_first_reject(k, vp(pa.ctypes.data), vp(qa.ctypes.data), vp(un.ctypes.data),
                                              ctypes.byref(pos)), "kq_speculative_first_reject")
    return int(pos.value)


def speculative_resample(p_row, q_row, order, u):
    """The token drawn where the decision stops (host arrays): from the
    residual of p_row and q_row, or from p_row alone when q_row is None."""
    import numpy as np
    p = np.ascontiguousarray(p_row, dtype=np.float32)
    n = int(p.shape[0])
    q = np.ascontiguousarray(q_row, dtype=np.float32) if q_row is not None else None
    od = np.ascontiguousarray(order, dtype=np.int32)
    if od.shape != (n,) or (q is not None and q.shape != (n,)):
        raise ValueError("p_row, q_row and order must have the same length")
    tok = ctypes.c_int32(0)
    vp = ctypes.c_void_p
    _check(load().kq_speculative_resample(n, vp(p.ctypes.data), vp(q.ctypes.data) if q is not None else None,
                                          vp(od.ctypes.data), ctypes.c_float(float(u)), ctypes.byref(tok)),
           "kq_speculative_resample")
    return int(tok.value)
