"""CPU oracle for the k-quant (Q4_K, Q5_K, Q6_K) batched verify step (ctypes
wrapper over kq_oracle.c).

TEST INFRASTRUCTURE ONLY. The product library never imports, links or runs
anything here; only tests/, the smoke check and the bench's CPU-baseline leg
do. It shares no code with the HIP path: its own fp16 decode, its own scale
unpacking, its own fp64 dot products.

What each function follows is stated in kq_oracle.c. Every function here is
pinned by CPU tests against hand-built blocks, exact rational arithmetic,
closed forms and brute-force enumeration (tests/test_oracle_*.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
_LIB = os.path.join(_HERE, "libkq_oracle.so")
_lib = None
_threads = 0  # OpenMP threads when the library was first loaded

REL_TOL = 1e-4  # declared logit tolerance: |G - L| <= REL_TOL * sum_k |w_k x_k|

# weight formats: name -> (code of the C functions, bytes per 256 weights)
FORMATS = {"q4k": (4, 144), "q5k": (5, 176), "q6k": (6, 210)}


def block_bytes(fmt: str = "q4k") -> int:
    return FORMATS[fmt][1]


def build(force: bool = True) -> str:
    """Compile kq_oracle.c with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib, _threads
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.kqo_half_to_double.argtypes = [ctypes.c_uint16]
    lib.kqo_half_to_double.restype = ctypes.c_double
    lib.kqo_scales_mins.argtypes = [P, P, P]
    lib.kqo_quant.argtypes = [P, ctypes.c_int]
    lib.kqo_quant.restype = ctypes.c_int
    lib.kqo_decode_block.argtypes = [P, P]
    lib.kqo_decode_block.restype = ctypes.c_int
    lib.kqo_decode_row.argtypes = [P, i64, P]
    lib.kqo_decode_row.restype = ctypes.c_int
    lib.kqo_gemv_rows.argtypes = [P, i64, i64, P, ctypes.c_int, P, i64, P, P, ctypes.c_int]
    lib.kqo_gemv_rows.restype = ctypes.c_int
    lib.kqo_argmax_flags.argtypes = [P, P, ctypes.c_int, i64, ctypes.c_double, P, P]
    lib.kqo_argmax_flags.restype = ctypes.c_int
    lib.kqo_candidates.argtypes = [P, P, i64, ctypes.c_int32, ctypes.c_double, P, i64]
    lib.kqo_candidates.restype = i64
    lib.kqo_accept.argtypes = [P, ctypes.c_int, P, P, P]
    lib.kqo_accept.restype = ctypes.c_int
    lib.kqo_quant_q5k.argtypes = [P, P, ctypes.c_int]
    lib.kqo_quant_q5k.restype = ctypes.c_int
    lib.kqo_quant_q6k.argtypes = [P, P, ctypes.c_int]
    lib.kqo_quant_q6k.restype = ctypes.c_int
    lib.kqo_decode_block_fmt.argtypes = [ctypes.c_int, P, P]
    lib.kqo_decode_block_fmt.restype = ctypes.c_int
    lib.kqo_decode_row_fmt.argtypes = [ctypes.c_int, P, i64, P]
    lib.kqo_decode_row_fmt.restype = ctypes.c_int
    lib.kqo_gemv_rows_fmt.argtypes = [ctypes.c_int, P, i64, i64, P, ctypes.c_int, P, i64, P, P, ctypes.c_int]
    lib.kqo_gemv_rows_fmt.restype = ctypes.c_int
    lib.kqo_tree_accept.argtypes = [P, P, ctypes.c_int, P, P, P, P]
    lib.kqo_tree_accept.restype = ctypes.c_int
    lib.kqo_term_mass_q4k.argtypes = [P, i64, i64, P, ctypes.c_int, P, i64, P]
    lib.kqo_term_mass_q4k.restype = ctypes.c_int
    lib.kqo_num_threads.argtypes = []
    lib.kqo_num_threads.restype = ctypes.c_int
    _threads = int(lib.kqo_num_threads())
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads a call with threads=0 uses: the OpenMP default when the
    library was first loaded (a call with an explicit count changes the
    OpenMP setting for later calls; this count does not follow it)."""
    _load()
    return _threads


def half_to_double(bits: int) -> float:
    return float(_load().kqo_half_to_double(int(bits) & 0xFFFF))


def scales_mins(s12: bytes) -> Tuple[np.ndarray, np.ndarray]:
    s = np.frombuffer(bytes(s12), dtype=np.uint8).copy()
    assert s.shape == (12,)
    sc = np.zeros(8, dtype=np.int32)
    mn = np.zeros(8, dtype=np.int32)
    _load().kqo_scales_mins(_p(s), _p(sc), _p(mn))
    return sc, mn


def decode_block(blk, fmt: str = "q4k") -> np.ndarray:
    """The 256 exact weights (fp64) of one block of format `fmt`."""
    code, nb = FORMATS[fmt]
    b = np.ascontiguousarray(np.frombuffer(bytes(blk), dtype=np.uint8))
    assert b.shape == (nb,)
    w = np.zeros(256, dtype=np.float64)
    if _load().kqo_decode_block_fmt(code, _p(b), _p(w)):
        raise ValueError("non-finite block scale")
    return w


def decode_matrix(w: np.ndarray, k: int, fmt: str = "q4k") -> np.ndarray:
    """Exact fp64 weights [N, K] of a matrix of format `fmt` (small matrices only)."""
    code, _ = FORMATS[fmt]
    w = np.ascontiguousarray(w, dtype=np.uint8)
    n = w.shape[0]
    out = np.zeros((n, k), dtype=np.float64)
    lib = _load()
    for r in range(n):
        row = np.ascontiguousarray(w[r])
        if lib.kqo_decode_row_fmt(code, _p(row), k, _p(out[r])):
            raise ValueError("non-finite block scale")
    return out


def gemv_rows(w: np.ndarray, k: int, x: np.ndarray, rows: Optional[Sequence[int]] = None,
              threads: int = 0, fmt: str = "q4k") -> Tuple[np.ndarray, np.ndarray]:
    """(L, A), each float64 [M, n_out]: L = W x^T in fp64, A = sum |w x|.

    w: uint8 [N, K/256 * block bytes of `fmt`]; x: float32 [M, K]; rows:
    optional subset of the N output rows (outputs then follow that order)."""
    code, nb = FORMATS[fmt]
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    n = w.shape[0]
    m = x.shape[0]
    if x.shape[1] != k or w.shape[1] != (k // 256) * nb:
        raise ValueError("shape mismatch")
    if rows is None:
        r_arr = None
        nout = n
    else:
        r_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nout = r_arr.shape[0]
    L = np.zeros((m, nout), dtype=np.float64)
    A = np.zeros((m, nout), dtype=np.float64)
    rc = _load().kqo_gemv_rows_fmt(code, _p(w), n, k, _p(x), m,
                                   _p(r_arr) if r_arr is not None else None, nout,
                                   _p(L), _p(A), int(threads) if threads > 0 else num_threads())
    if rc == -3:
        raise ValueError("non-finite activation")
    if rc == -2:
        raise ValueError("non-finite block scale")
    if rc:
        raise ValueError("bad shape")
    return L, A


def term_mass(w: np.ndarray, k: int, x: np.ndarray, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """B, float64 [M, n_out]: sum_k (|d sc_j q_k| + |dmin m_j|) |x_k| for a
    Q4_K matrix (kqo_term_mass_q4k), the mass the rounding error of a kernel
    that forms a block's scale and min terms apart is proportional to."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    n, m = w.shape[0], x.shape[0]
    if x.shape[1] != k or w.shape[1] != (k // 256) * 144:
        raise ValueError("shape mismatch")
    r_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nout = n if r_arr is None else r_arr.shape[0]
    B = np.zeros((m, nout), dtype=np.float64)
    rc = _load().kqo_term_mass_q4k(_p(w), n, k, _p(x), m, _p(r_arr) if r_arr is not None else None, nout, _p(B))
    if rc == -3:
        raise ValueError("non-finite activation")
    if rc == -2:
        raise ValueError("non-finite block scale")
    if rc:
        raise ValueError("bad shape")
    return B


def argmax_flags(L: np.ndarray, A: np.ndarray, rel: float = REL_TOL) -> Tuple[np.ndarray, np.ndarray]:
    L = np.ascontiguousarray(L, dtype=np.float64)
    A = np.ascontiguousarray(A, dtype=np.float64)
    m, n = L.shape
    am = np.zeros(m, dtype=np.int32)
    nc = np.zeros(m, dtype=np.int64)
    if _load().kqo_argmax_flags(_p(L), _p(A), m, n, float(rel), _p(am), _p(nc)):
        raise ValueError("bad shape")
    return am, nc


def candidates(L_row: np.ndarray, A_row: np.ndarray, best: int, rel: float = REL_TOL) -> np.ndarray:
    L_row = np.ascontiguousarray(L_row, dtype=np.float64)
    A_row = np.ascontiguousarray(A_row, dtype=np.float64)
    n = L_row.shape[0]
    lib = _load()
    cnt = lib.kqo_candidates(_p(L_row), _p(A_row), n, int(best), float(rel), None, 0)
    out = np.zeros(max(cnt, 1), dtype=np.int32)
    lib.kqo_candidates(_p(L_row), _p(A_row), n, int(best), float(rel), _p(out), cnt)
    return out[:cnt]


def accept(draft: Sequence[int], argmax: Sequence[int]) -> Tuple[int, int]:
    d = np.ascontiguousarray(np.asarray(draft, dtype=np.int32))
    a = np.ascontiguousarray(np.asarray(argmax, dtype=np.int32))
    k = d.shape[0]
    if a.shape[0] != k + 1:
        raise ValueError("need k+1 target rows for k draft tokens")
    acc = ctypes.c_int32(0)
    nxt = ctypes.c_int32(0)
    _load().kqo_accept(_p(d) if k else None, k, _p(a), ctypes.byref(acc), ctypes.byref(nxt))
    return int(acc.value), int(nxt.value)


def tree_accept(parent: Sequence[int], token: Sequence[int], argmax: Sequence[int]) -> Tuple[int, int, list]:
    """(accepted, next_token, path) of the greedy walk over a token tree
    (kqo_tree_accept): parent[0] = -1, parent[j] < j, token[j] the token node
    j proposes, argmax[j] the target's argmax of row j."""
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    tok = np.ascontiguousarray(np.asarray(token, dtype=np.int32))
    am = np.ascontiguousarray(np.asarray(argmax, dtype=np.int32))
    m = par.shape[0]
    if tok.shape[0] != m or am.shape[0] != m:
        raise ValueError("parent, token and argmax need one entry per node")
    acc, nxt = ctypes.c_int32(0), ctypes.c_int32(0)
    path = np.zeros(max(m, 1), dtype=np.int32)
    if _load().kqo_tree_accept(_p(par), _p(tok), m, _p(am), ctypes.byref(acc), ctypes.byref(nxt), _p(path)):
        raise ValueError("invalid tree: parent[0] must be -1 and parent[j] in [0, j)")
    return int(acc.value), int(nxt.value), [int(v) for v in path[:acc.value]]


def verify(w: np.ndarray, k: int, x: np.ndarray, draft: Sequence[int], rel: float = REL_TOL,
           threads: int = 0, fmt: str = "q4k"):
    """The whole step on the CPU: logits, argmax with flags, greedy accept.
    Returns dict(L, A, argmax, n_cand, accepted, next_token)."""
    L, A = gemv_rows(w, k, x, threads=threads, fmt=fmt)
    am, nc = argmax_flags(L, A, rel)
    acc, nxt = accept(draft, am)
    return dict(L=L, A=A, argmax=am, n_cand=nc, accepted=acc, next_token=nxt)
