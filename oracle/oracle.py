"""ctypes front of the plain C oracle (w4moe_oracle.c).

TEST INFRASTRUCTURE, NOT THE PRODUCT: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this. It does not import the HIP package and the HIP package does not
import it.

Functions:
  moe_forward(dims, x, ids, w, experts, rows=None, nthreads=0) -> float64 [n_rows, K]
      the layer output (fp32 dequantisation, fp64 sums, no rounding), for the listed token rows.
      experts[e] is (w1, s1, w2, s2), or (w1, s1, w2, s2, g_idx1, g_idx2) for activation-ordered
      weights (the scale row of every reduction row given explicitly).
  moe_align(ids, E, B) -> dict(counts, offsets, sorted_ids, block_expert, active)
      stable padded token-to-expert sort of the flat routing entries.
  expert_ffn(dims, xrow, w1, s1, w2, s2, g1=None, g2=None) -> float64 [K]
                                                          one SwiGLU expert on one token.
  code(wq, r, c, bits=4) / dequant(wq, sc, group, r, c, bits=4)
                                                          single-element unpack / dequantisation
                                                          (4-bit codes 8 per int32, or 8-bit 4 per int32).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

__all__ = ["load", "moe_forward", "moe_align", "expert_ffn", "code", "dequant", "ORACLE_LIB"]

ORACLE_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4moe_oracle.so")
_lib = None


class _Dims(C.Structure):
    _fields_ = [("E", C.c_int32), ("K", C.c_int32), ("N", C.c_int32), ("topk", C.c_int32), ("group", C.c_int32),
                ("bits", C.c_int32)]


def load():
    """Load the compiled oracle, building it first if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(ORACLE_LIB):
            from . import build as _b
            _b.build()
        lib = C.CDLL(ORACLE_LIB)
        P = C.c_void_p
        lib.w4o_moe_forward.argtypes = [C.POINTER(_Dims), C.c_int32, P, P, P, P, P, P, P, P, P, C.c_int32, P, P,
                                        C.c_int32]
        lib.w4o_moe_forward.restype = C.c_int
        lib.w4o_moe_align.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, P, P, C.c_int32, P, C.c_int32, P, P]
        lib.w4o_moe_align.restype = C.c_int32
        lib.w4o_expert_ffn.argtypes = [C.POINTER(_Dims), P, P, P, P, P, P, P, P, P]
        lib.w4o_expert_ffn.restype = None
        lib.w4o_code.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, C.c_int32]
        lib.w4o_code.restype = C.c_int
        lib.w4o_dequant.argtypes = [P, P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32]
        lib.w4o_dequant.restype = C.c_float
        _lib = lib
    return _lib


def _dims(d):
    return _Dims(d.E, d.K, d.N, d.topk, d.group, getattr(d, "bits", 4))


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def moe_forward(dims, x, ids, w, experts, rows=None, nthreads=0):
    """x: bf16 bits [M, K]; ids int32 [M, k]; w float32 [M, k]; experts: mapping e -> (w1, s1, w2, s2)
    in the logical layout, or (w1, s1, w2, s2, g_idx1, g_idx2) with activation order (only routed
    experts of the listed rows are needed)."""
    lib = load()
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    M = x.shape[0]
    assert x.shape == (M, dims.K) and ids.shape == (M, dims.topk) and w.shape == ids.shape
    rows_arr = None if rows is None else _c(rows, np.int32)
    n_rows = M if rows_arr is None else int(rows_arr.size)
    needed = np.unique(ids if rows_arr is None else ids[rows_arr]) if n_rows else np.zeros(0, np.int32)
    keep = []
    arrs = [(C.c_void_p * dims.E)() for _ in range(6)]
    for e in needed:
        e = int(e)
        if not (0 <= e < dims.E):
            raise ValueError(f"expert id {e} out of range")
        parts = experts[e]
        for i, (arr, dt) in enumerate(zip(parts, (np.int32, np.uint16, np.int32, np.uint16, np.int32, np.int32))):
            a = _c(arr, dt)
            keep.append(a)
            arrs[i][e] = a.ctypes.data
    out = np.zeros((n_rows, dims.K), dtype=np.float64)
    rc = lib.w4o_moe_forward(C.byref(_dims(dims)), M, _ptr(x), _ptr(ids), _ptr(w),
                             C.cast(arrs[0], C.c_void_p), C.cast(arrs[1], C.c_void_p),
                             C.cast(arrs[2], C.c_void_p), C.cast(arrs[3], C.c_void_p),
                             C.cast(arrs[4], C.c_void_p), C.cast(arrs[5], C.c_void_p),
                             n_rows, None if rows_arr is None else _ptr(rows_arr), _ptr(out), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"w4o_moe_forward failed with code {rc}")
    return out


def moe_align(ids, E, B):
    """Stable padded sort of the flat routing entries of ids (any shape, flattened row-major)."""
    lib = load()
    flat = _c(np.asarray(ids).reshape(-1), np.int32)
    T = int(flat.size)
    cap = T + min(E, T) * (B - 1) + 1
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_ids = np.zeros(cap, np.int32)
    block_expert = np.zeros(cap // B + 1, np.int32)
    active = np.zeros(E, np.int32)
    n_active = np.zeros(1, np.int32)
    P = lib.w4o_moe_align(T, E, B, _ptr(flat), _ptr(counts), _ptr(offsets), _ptr(sorted_ids), cap,
                          _ptr(block_expert), block_expert.size, _ptr(active), _ptr(n_active))
    if P < 0:
        raise RuntimeError(f"w4o_moe_align failed with code {P}")
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids[:P], block_expert=block_expert[:P // B],
                active=active[:int(n_active[0])], padded_rows=int(P))


def expert_ffn(dims, xrow, w1, s1, w2, s2, g1=None, g2=None):
    """One SwiGLU expert on one token (bf16 bits [K]) -> float64 [K]; g1 [K] / g2 [N] are the group
    indices of activation-ordered weights (None: consecutive groups)."""
    lib = load()
    xrow = _c(xrow, np.uint16)
    arrs = [_c(w1, np.int32), _c(s1, np.uint16), _c(w2, np.int32), _c(s2, np.uint16)]
    gs = [None if g is None else _c(g, np.int32) for g in (g1, g2)]
    for g, R in zip(gs, (dims.K, dims.N)):
        if g is not None and (g.shape != (R,) or g.min() < 0 or g.max() >= R // dims.group):
            raise ValueError("group index out of range")
    h = np.zeros(2 * dims.N, np.float64)
    y = np.zeros(dims.K, np.float64)
    lib.w4o_expert_ffn(C.byref(_dims(dims)), _ptr(xrow), *[_ptr(a) for a in arrs],
                       *[None if g is None else _ptr(g) for g in gs], _ptr(h), _ptr(y))
    return y


def code(wq, r, c, bits=4):
    wq = _c(wq, np.int32)
    return load().w4o_code(_ptr(wq), wq.shape[1], int(bits), int(r), int(c))


def dequant(wq, sc, group, r, c, bits=4):
    wq = _c(wq, np.int32)
    sc = _c(sc, np.uint16)
    return load().w4o_dequant(_ptr(wq), _ptr(sc), wq.shape[1], int(bits), int(group), int(r), int(c))
