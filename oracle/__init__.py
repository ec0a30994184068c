"""fp64 CPU oracle for NSA selection attention (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
bench's CPU-baseline leg, never by the GPU library or its binding.  It shares
no code with the GPU path; both only consume arrays made by the seeded input
generator.

The arithmetic lives in ``nsa_oracle.c`` (plain C, fp64, exact two-pass
softmax over the union of selected, causally visible keys); this module only
loads it and marshals numpy arrays.  Its header lists the page sections it
follows and the readings taken where the page is silent.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB = os.path.join(_HERE, "libnsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, -O2)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.nsa_oracle_half_to_double.restype = ctypes.c_double
        lib.nsa_oracle_half_to_double.argtypes = [ctypes.c_uint16]
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.nsa_oracle_units.restype = ctypes.c_int
        lib.nsa_oracle_units.argtypes = [p, p, p, p] + [i64] * 8 + [p, i64, p, p, p, ctypes.c_int]
        lib.nsa_oracle_dense_units.restype = ctypes.c_int
        lib.nsa_oracle_dense_units.argtypes = [p, p, p] + [i64] * 6 + [p, i64, p, p, ctypes.c_int]
        lib.nsa_oracle_bf16_to_double.restype = ctypes.c_double
        lib.nsa_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.nsa_oracle_units_t.restype = ctypes.c_int
        lib.nsa_oracle_units_t.argtypes = [p, p, p, p] + [i64] * 8 + [p, i64, p, p, p, ctypes.c_int, ctypes.c_int]
        lib.nsa_oracle_window_units.restype = ctypes.c_int
        lib.nsa_oracle_window_units.argtypes = ([p, p, p] + [i64] * 8 + [p, i64, p, p, ctypes.c_int, ctypes.c_int])
        lib.nsa_oracle_bwd_units.restype = ctypes.c_int
        lib.nsa_oracle_bwd_units.argtypes = ([p] * 5 + [i64] * 8 + [p, i64, p, i64, p, p, p, p, p, p, ctypes.c_int])
        lib.nsa_oracle_compare.restype = ctypes.c_int
        lib.nsa_oracle_compare.argtypes = ([p] * 4 + [i64] * 10 + [p, p, i64, i64, ctypes.c_int, ctypes.c_int, p])
        lib.nsa_oracle_topk.restype = ctypes.c_int
        lib.nsa_oracle_topk.argtypes = [p] + [i64] * 6 + [p]
        lib.nsa_oracle_topk_rows.restype = ctypes.c_int
        lib.nsa_oracle_topk_rows.argtypes = [p, p] + [i64] * 4 + [p]
        _lib = lib
    return _lib


def half_to_double(bits: int) -> float:
    return _load().nsa_oracle_half_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return _load().nsa_oracle_bf16_to_double(bits)


# Element types: fp16 arrays are numpy float16; bf16 arrays are numpy uint16
# holding the bfloat16 bit patterns (numpy has no bfloat16 type).
_ELEM = {"fp16": (np.float16, 0), "bf16": (np.uint16, 1)}


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _check_inputs(q, k, v, idx, dtype="fp16"):
    et = _ELEM[dtype][0]
    for name, a, dt in (("Q", q, et), ("K", k, et), ("V", v, et),
                        ("block_indices", idx, np.int32)):
        if a.dtype != dt or not a.flags.c_contiguous or a.ndim != 4:
            raise ValueError(f"{name} must be a C-contiguous 4-d {np.dtype(dt).name} array")
    B, M, H, D = q.shape
    Bk, N, G, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or idx.shape[:3] != (B, M, G) or H % G:
        raise ValueError("inconsistent shapes")
    return B, M, N, H, G, D, idx.shape[3]


def oracle_units(q, k, v, idx, block_size: int, units: np.ndarray, threads: int = 0, dtype: str = "fp16"):
    """O (fp64 [U, H/G, D]) and LSE (fp64 [U, H/G]) for units (b, m, g).
    dtype "bf16" takes Q, K, V as uint16 arrays of bfloat16 bit patterns."""
    B, M, N, H, G, D, T = _check_inputs(q, k, v, idx, dtype)
    units = np.ascontiguousarray(units, dtype=np.int64).reshape(-1, 3)
    U = units.shape[0]
    gs = H // G
    O = np.empty((U, gs, D), dtype=np.float64)
    L = np.empty((U, gs), dtype=np.float64)
    ndup = ctypes.c_int64(0)
    rc = _load().nsa_oracle_units_t(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), B, M, N, H, G, D,
                                    block_size, T, _ptr(units), U, _ptr(O), _ptr(L),
                                    ctypes.byref(ndup), _ELEM[dtype][1], threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    oracle_units.last_dup_units = ndup.value
    return O, L


oracle_units.last_dup_units = 0


def all_units(B: int, M: int, G: int) -> np.ndarray:
    b, m, g = np.meshgrid(np.arange(B), np.arange(M), np.arange(G), indexing="ij")
    return np.stack([b.ravel(), m.ravel(), g.ravel()], axis=1).astype(np.int64)


def oracle_full(q, k, v, idx, block_size: int, threads: int = 0, dtype: str = "fp16"):
    """Whole-tensor oracle: O fp64 [B, M, H, D] and LSE fp64 [B, H, M]."""
    B, M, N, H, G, D, T = _check_inputs(q, k, v, idx, dtype)
    O, L = oracle_units(q, k, v, idx, block_size, all_units(B, M, G), threads, dtype)
    O = O.reshape(B, M, H, D)
    L = L.reshape(B, M, H).transpose(0, 2, 1).copy()
    return O, L


def dense_units(q, k, v, units: np.ndarray, threads: int = 0):
    """Dense causal attention (every key n <= m, n < N visible) for units
    (b, m, g): O fp64 [U, H/G, D] and LSE fp64 [U, H/G].  The same fp64
    two-pass computation as ``oracle_units`` without an index array."""
    idx = np.zeros((q.shape[0], q.shape[1], k.shape[2], 1), np.int32)
    B, M, N, H, G, D, _ = _check_inputs(q, k, v, idx)
    units = np.ascontiguousarray(units, dtype=np.int64).reshape(-1, 3)
    U = units.shape[0]
    gs = H // G
    O = np.empty((U, gs, D), dtype=np.float64)
    L = np.empty((U, gs), dtype=np.float64)
    rc = _load().nsa_oracle_dense_units(_ptr(q), _ptr(k), _ptr(v), B, M, N, H, G, D, _ptr(units), U, _ptr(O),
                                        _ptr(L), threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return O, L


def window_units(q, k, v, left: int, right: int, units: np.ndarray, threads: int = 0, dtype: str = "fp16"):
    """Sliding-window attention for units (b, m, g): keys n < N with
    m - left <= n <= m + right (negative = unbounded on that side);
    O fp64 [U, H/G, D], LSE fp64 [U, H/G]."""
    idx = np.zeros((q.shape[0], q.shape[1], k.shape[2], 1), np.int32)
    B, M, N, H, G, D, _ = _check_inputs(q, k, v, idx, dtype)
    units = np.ascontiguousarray(units, dtype=np.int64).reshape(-1, 3)
    U = units.shape[0]
    gs = H // G
    O = np.empty((U, gs, D), dtype=np.float64)
    L = np.empty((U, gs), dtype=np.float64)
    rc = _load().nsa_oracle_window_units(_ptr(q), _ptr(k), _ptr(v), B, M, N, H, G, D, left, right, _ptr(units), U,
                                         _ptr(O), _ptr(L), _ELEM[dtype][1], threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return O, L


def window_full(q, k, v, left: int, right: int, threads: int = 0, dtype: str = "fp16"):
    """Whole-tensor sliding-window attention: O fp64 [B, M, H, D], LSE fp64 [B, H, M]."""
    B, M, H, D = q.shape
    G = k.shape[2]
    O, L = window_units(q, k, v, left, right, all_units(B, M, G), threads, dtype)
    return O.reshape(B, M, H, D), L.reshape(B, M, H).transpose(0, 2, 1).copy()


def dense_full(q, k, v, threads: int = 0):
    """Whole-tensor dense causal attention: O fp64 [B, M, H, D], LSE fp64 [B, H, M]."""
    B, M, H, D = q.shape
    G = k.shape[2]
    O, L = dense_units(q, k, v, all_units(B, M, G), threads)
    return O.reshape(B, M, H, D), L.reshape(B, M, H).transpose(0, 2, 1).copy()


def compare(q, k, v, idx, block_size: int, O, L, u0: int = 0, u1: int | None = None, threads: int = 0,
            dtype: str = "fp16", window: tuple[int, int] | None = None) -> dict:
    """Compares a computed forward result O [B, M, H, D] (fp16, or bf16 bit
    patterns as uint16) and LSE L fp32 [B, H, M] with the oracle over the units
    u0 .. u1-1 of the order u = (b*M + m)*G + g, one unit at a time (no fp64
    copy of the outputs is kept).  idx None compares with the attention
    without index rows over ``window`` = (left, right) (default (-1, 0): dense
    causal).  Returns max_err_O (every element; an empty row's reference is
    0), max_err_LSE (rows with a finite reference), bad_rows (non-finite O or
    LSE where the reference is finite, or LSE != -inf on an empty row), the
    units holding the largest errors, units compared, units with repeated
    blocks and empty rows."""
    if idx is None:
        idx_arr = np.zeros((q.shape[0], q.shape[1], k.shape[2], 1), np.int32)
    else:
        idx_arr = idx
    B, M, N, H, G, D, T = _check_inputs(q, k, v, idx_arr, dtype)
    et = _ELEM[dtype][0]
    if O.dtype != et or O.shape != q.shape or not O.flags.c_contiguous:
        raise ValueError("O must be a C-contiguous array shaped and typed like Q")
    if L.dtype != np.float32 or L.shape != (B, H, M) or not L.flags.c_contiguous:
        raise ValueError("L must be a C-contiguous float32 [B, H, M] array")
    left, right = window if window is not None else (-1, 0)
    if u1 is None:
        u1 = B * M * G
    stats = np.zeros(8, dtype=np.float64)
    rc = _load().nsa_oracle_compare(_ptr(q), _ptr(k), _ptr(v), None if idx is None else _ptr(idx_arr), B, M, N, H,
                                    G, D, block_size, T, left, right, _ptr(O), _ptr(L), int(u0), int(u1),
                                    _ELEM[dtype][1], threads, _ptr(stats))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"max_err_O": float(stats[0]), "max_err_LSE": float(stats[1]), "bad_rows": int(stats[2]),
            "worst_unit_O": int(stats[3]), "worst_unit_LSE": int(stats[4]), "units": int(stats[5]),
            "dup_units": int(stats[6]), "empty_rows": int(stats[7])}


def bwd_units(q, k, v, idx, do, block_size: int, units: np.ndarray, kblocks: np.ndarray | None = None,
              threads: int = 0, mags: bool = False):
    """Gradients of the selection attention of units (b, m, g) for the upstream
    gradient ``do`` (fp16 [B, M, H, D]).

    idx None means dense causal attention (every key n <= m visible).
    Returns dQ fp64 [U, H/G, D] for the units, and dK, dV fp64 summed over the
    units: [B, N, G, D] when ``kblocks`` is None, else [n_kblocks, bs, D] for
    the key blocks (b, g, t) listed there (rows past N stay zero).  Only the
    given units contribute, so a key block's dK/dV is complete when every unit
    that selects it is listed.

    mags=True also returns, laid out like dQ, dK, dV, the L2 norm over each
    element's terms of the term magnitudes (dS taken as P (|dP| + sum_d |dO_d
    O_d|)): the scale of the rounding error of a kernel that rounds P, dS and
    the O that Delta is formed from."""
    if idx is None:
        idx_arr = np.zeros((q.shape[0], q.shape[1], k.shape[2], 1), np.int32)
    else:
        idx_arr = idx
    B, M, N, H, G, D, T = _check_inputs(q, k, v, idx_arr)
    if do.dtype != np.float16 or not do.flags.c_contiguous or do.shape != q.shape:
        raise ValueError("dO must be a C-contiguous float16 array shaped like Q")
    units = np.ascontiguousarray(units, dtype=np.int64).reshape(-1, 3)
    U = units.shape[0]
    gs = H // G
    dQ = np.empty((U, gs, D), dtype=np.float64)
    if kblocks is None:
        kb_ptr, nkb = None, 0
        dK = np.zeros((B, N, G, D), dtype=np.float64)
    else:
        kblocks = np.ascontiguousarray(kblocks, dtype=np.int64).reshape(-1, 3)
        kb_ptr, nkb = _ptr(kblocks), kblocks.shape[0]
        dK = np.zeros((nkb, block_size, D), dtype=np.float64)
    dV = np.zeros_like(dK)
    if mags:
        mQ, mK, mV = np.empty_like(dQ), np.zeros_like(dK), np.zeros_like(dK)
        mp = (_ptr(mQ), _ptr(mK), _ptr(mV))
    else:
        mp = (None, None, None)
    rc = _load().nsa_oracle_bwd_units(_ptr(q), _ptr(k), _ptr(v), None if idx is None else _ptr(idx_arr), _ptr(do),
                                      B, M, N, H, G, D, block_size, T, _ptr(units), U, kb_ptr, nkb,
                                      _ptr(dQ), _ptr(dK), _ptr(dV), *mp, threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if mags:
        return dQ, dK, dV, mQ, mK, mV
    return dQ, dK, dV


def bwd_full(q, k, v, idx, do, block_size: int, threads: int = 0, mags: bool = False):
    """Whole-tensor gradients: dQ fp64 [B, M, H, D], dK and dV fp64 [B, N, G, D]
    (and with mags=True their term magnitudes, laid out alike)."""
    B, M, H, D = q.shape
    G = k.shape[2]
    r = bwd_units(q, k, v, idx, do, block_size, all_units(B, M, G), None, threads, mags)
    out = [r[0].reshape(B, M, H, D), r[1], r[2]]
    if mags:
        out += [r[3].reshape(B, M, H, D), r[4], r[5]]
    return tuple(out)


def topk_blocks(scores: np.ndarray, block_size: int, T: int) -> np.ndarray:
    """Top-k block selection: scores fp32 [B, M, G, NB] -> block_indices int32
    [B, M, G, T].  Per row, the T highest-scoring blocks among t = 0 ..
    min(m // block_size, NB - 1) (ties: smaller t first; NaN counts as -inf),
    written in ascending order, padded with -1."""
    if scores.dtype != np.float32 or scores.ndim != 4 or not scores.flags.c_contiguous:
        raise ValueError("scores must be a C-contiguous 4-d float32 array")
    B, M, G, NB = scores.shape
    out = np.empty((B, M, G, T), dtype=np.int32)
    if _load().nsa_oracle_topk(_ptr(scores), B, M, G, NB, block_size, T, _ptr(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def topk_rows(scores_rows: np.ndarray, ms: np.ndarray, block_size: int, T: int) -> np.ndarray:
    """topk_blocks for explicit rows: scores fp32 [R, NB] of queries at
    positions ms [R] -> int32 [R, T]."""
    scores_rows = np.ascontiguousarray(scores_rows, dtype=np.float32)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    R, NB = scores_rows.shape
    out = np.empty((R, T), dtype=np.int32)
    if _load().nsa_oracle_topk_rows(_ptr(scores_rows), _ptr(ms), R, NB, block_size, T, _ptr(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out
