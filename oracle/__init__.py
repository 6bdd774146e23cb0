"""CPU oracle for the expert-ID matmul path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product path (the HIP library and its binding) never
imports it.  The arithmetic lives in eidm_oracle.c (plain C, double
precision); this module compiles it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eidm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, F16, BF16 = 0, 1, 2
SHARED, SLOTTED = 0, 1


def build() -> str:
    """Compile the oracle (no fast-math, no contraction: every operation is
    the one written)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Werror", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    u32, u64, i32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
    lib.oracle_widen.restype = ctypes.c_double
    lib.oracle_widen.argtypes = [i32, P]
    lib.oracle_required_weight_bytes.restype = u64
    lib.oracle_required_weight_bytes.argtypes = [i32, u32, u32, u32, u64]
    lib.oracle_route.restype = i32
    lib.oracle_route.argtypes = [P, P, u32, u32, u32, i32, P, P, P, P]
    lib.oracle_matmul_id.restype = i32
    lib.oracle_matmul_id.argtypes = [i32, u32, u32, u32, u32, u32, u64, i32, P, P, P, P]
    lib.oracle_matmul_id_threads.restype = i32
    lib.oracle_matmul_id_threads.argtypes = [i32, u32, u32, u32, u32, u32, u64, i32, P, P, P, P, i32]
    lib.oracle_matmul_id_at.restype = i32
    lib.oracle_matmul_id_at.argtypes = [i32, u32, u32, u32, u32, u32, u64, i32, P, P, P, u64, P, P, P]
    lib.oracle_combine.restype = i32
    lib.oracle_combine.argtypes = [u32, u32, u32, P, P, P]
    lib.oracle_moe_ffn.restype = i32
    lib.oracle_moe_ffn.argtypes = [i32, u32, u32, u32, u32, u32, u64, u64, P, P, P, P, P, P, P, P]
    lib.oracle_map.restype = i32
    lib.oracle_map.argtypes = [P, u64, u32, P, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def widen(dtype: int, raw: bytes) -> float:
    buf = np.frombuffer(raw, dtype=np.uint8).copy()
    return _load().oracle_widen(dtype, _ptr(buf))


def widen_array(dtype: int, bits: np.ndarray) -> np.ndarray:
    """Widen every element of a uint16/uint32 bit array (slow: one call each)."""
    lib = _load()
    flat = np.ascontiguousarray(bits).reshape(-1)
    out = np.empty(flat.size, dtype=np.float64)
    itemsize = flat.dtype.itemsize
    base = flat.ctypes.data
    for i in range(flat.size):
        out[i] = lib.oracle_widen(dtype, ctypes.c_void_p(base + i * itemsize))
    return out.reshape(bits.shape)


def required_weight_bytes(dtype: int, n: int, k: int, n_experts: int, stride: int) -> int:
    return int(_load().oracle_required_weight_bytes(dtype, n, k, n_experts, stride))


def route(logits: np.ndarray, bias: np.ndarray | None, top_k: int, renormalize: bool = True):
    """-> (ids u32 [m,top_k], gates f64 [m,top_k], sigma f32 [m,E], sel f32 [m,E])."""
    logits = _c(logits, np.float32)
    m, n_experts = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((m, top_k), dtype=np.uint32)
    gates = np.empty((m, top_k), dtype=np.float64)
    sigma = np.empty((m, n_experts), dtype=np.float32)
    sel = np.empty((m, n_experts), dtype=np.float32)
    rc = _load().oracle_route(_ptr(logits), _ptr(b), m, n_experts, top_k, int(renormalize),
                              _ptr(ids), _ptr(gates), _ptr(sigma), _ptr(sel))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return ids, gates, sigma, sel


def matmul_id(dtype: int, m: int, n: int, k: int, top_k: int, n_experts: int, stride: int,
              layout: int, weights: np.ndarray, x: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """y f64 [m*top_k, n]; weights is the raw byte buffer."""
    w = _c(weights, np.uint8).reshape(-1)
    assert w.size >= required_weight_bytes(dtype, n, k, n_experts, stride)
    x = _c(x, np.float32)
    ids = _c(ids, np.uint32)
    rows_in = m * top_k if layout == SLOTTED else m
    assert x.size == rows_in * k and ids.size == m * top_k
    y = np.empty((m * top_k, n), dtype=np.float64)
    rc = _load().oracle_matmul_id(dtype, m, n, k, top_k, n_experts, stride, layout,
                                  _ptr(w), _ptr(x), _ptr(ids), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle_matmul_id failed ({rc})")
    return y


def matmul_id_threads(dtype: int, m: int, n: int, k: int, top_k: int, n_experts: int, stride: int,
                      layout: int, weights: np.ndarray, x: np.ndarray, ids: np.ndarray,
                      threads: int) -> np.ndarray:
    """matmul_id split over `threads` host threads (the same values)."""
    w = _c(weights, np.uint8).reshape(-1)
    assert w.size >= required_weight_bytes(dtype, n, k, n_experts, stride)
    x = _c(x, np.float32)
    ids = _c(ids, np.uint32)
    rows_in = m * top_k if layout == SLOTTED else m
    assert x.size == rows_in * k and ids.size == m * top_k
    y = np.empty((m * top_k, n), dtype=np.float64)
    rc = _load().oracle_matmul_id_threads(dtype, m, n, k, top_k, n_experts, stride, layout,
                                          _ptr(w), _ptr(x), _ptr(ids), _ptr(y), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_matmul_id_threads failed ({rc})")
    return y


def matmul_id_at(dtype: int, m: int, n: int, k: int, top_k: int, n_experts: int, stride: int,
                 layout: int, weights: np.ndarray, x: np.ndarray, ids: np.ndarray,
                 rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """y[rows[i], cols[i]] in f64 for spot checks."""
    w = _c(weights, np.uint8).reshape(-1)
    x = _c(x, np.float32)
    ids = _c(ids, np.uint32)
    rows = _c(rows, np.uint64)
    cols = _c(cols, np.uint32)
    out = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_matmul_id_at(dtype, m, n, k, top_k, n_experts, stride, layout,
                                     _ptr(w), _ptr(x), _ptr(ids), rows.size, _ptr(rows),
                                     _ptr(cols), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_matmul_id_at failed ({rc})")
    return out


def combine(y: np.ndarray, gates: np.ndarray, top_k: int) -> np.ndarray:
    y = _c(y, np.float64)
    gates = _c(gates, np.float64)
    rows, n = y.shape
    m = rows // top_k
    out = np.empty((m, n), dtype=np.float64)
    _load().oracle_combine(m, top_k, n, _ptr(y), _ptr(gates), _ptr(out))
    return out


def id_map(ids: np.ndarray, n_experts: int):
    """-> (counts [E+1], offsets [E+2], rows [R]) of the stable sort by expert."""
    ids = _c(ids, np.uint32).reshape(-1)
    counts = np.empty(n_experts + 1, dtype=np.uint32)
    offsets = np.empty(n_experts + 2, dtype=np.uint32)
    rows = np.empty(ids.size, dtype=np.uint32)
    _load().oracle_map(_ptr(ids), ids.size, n_experts, _ptr(counts), _ptr(offsets), _ptr(rows))
    return counts, offsets, rows


def moe_ffn(dtype: int, m: int, hidden: int, inter: int, top_k: int, n_experts: int,
            gu_stride: int, down_stride: int, w_gate: np.ndarray, w_up: np.ndarray,
            w_down: np.ndarray, x: np.ndarray, ids: np.ndarray, gates: np.ndarray):
    """-> (out f64 [m, hidden], h f64 [m*top_k, inter]) of the expert FFN."""
    wg = _c(w_gate, np.uint8).reshape(-1)
    wu = _c(w_up, np.uint8).reshape(-1)
    wd = _c(w_down, np.uint8).reshape(-1)
    assert wg.size >= required_weight_bytes(dtype, inter, hidden, n_experts, gu_stride)
    assert wu.size >= required_weight_bytes(dtype, inter, hidden, n_experts, gu_stride)
    assert wd.size >= required_weight_bytes(dtype, hidden, inter, n_experts, down_stride)
    x = _c(x, np.float32)
    ids = _c(ids, np.uint32)
    gates = _c(gates, np.float64)
    assert x.size == m * hidden and ids.size == m * top_k and gates.size == m * top_k
    out = np.empty((m, hidden), dtype=np.float64)
    h = np.empty((m * top_k, inter), dtype=np.float64)
    rc = _load().oracle_moe_ffn(dtype, m, hidden, inter, top_k, n_experts, gu_stride, down_stride,
                                _ptr(wg), _ptr(wu), _ptr(wd), _ptr(x), _ptr(ids), _ptr(gates),
                                _ptr(h), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_moe_ffn failed ({rc})")
    return out, h
