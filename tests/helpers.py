"""Shared test helpers: device buffers, the tolerance check, the output
poison/guard check and the CPU canonical-order evaluator."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))

# max |gpu - oracle| / max(1, |oracle|), per element
TOL = 2e-5
# renormalised gates: f32 sum of top_k values and one f32 division
GATE_TOL = 2e-6

# the calibration proof's output poison and guard (mlx-native
# dense_matmul_id_auto.rs: fn poison_output / fn verified_bits)
POISON_BITS = 0x7FC000C7
GUARD = 16


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    nan_g, nan_r = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), "NaN positions differ"
    if (~nan_r).sum() == 0:
        return 0.0
    d = np.abs(gpu[~nan_r] - ref[~nan_r]) / np.maximum(1.0, np.abs(ref[~nan_r]))
    return float(d.max())


def assert_close(gpu, ref, tol=TOL, what=""):
    e = rel_err(gpu, ref)
    assert e <= tol, f"{what}: max rel err {e:.3e} > {tol:.1e}"
    return e


def poisoned_output(elements: int, device="cuda") -> torch.Tensor:
    t = torch.empty(elements + GUARD, dtype=torch.int32, device=device)
    t.fill_(POISON_BITS)
    return t.view(torch.float32)


def check_guarded(out: torch.Tensor, elements: int, allow_nan_rows: bool = False) -> np.ndarray:
    """Every logical element overwritten (finite unless allowed), guard untouched."""
    bits = out.view(torch.int32).cpu().numpy()
    body, guard = bits[:elements], bits[elements:]
    assert (guard == POISON_BITS).all(), "output guard was overwritten"
    assert not (body == POISON_BITS).any(), "an output element was not written"
    vals = body.view(np.float32)
    if not allow_nan_rows:
        assert np.isfinite(vals).all(), "non-finite output"
    return vals


_canon = None


def _canonical_lib():
    global _canon
    if _canon is None:
        src = os.path.join(HERE, "canonical_f32.c")
        so = os.path.join(HERE, "_canonical_f32.so")
        if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
            subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                            "-fno-fast-math", "-pthread", src, "-o", so + ".tmp", "-lm"], check=True)
            os.replace(so + ".tmp", so)
        lib = ctypes.CDLL(so)
        P = ctypes.c_void_p
        u32 = ctypes.c_uint32
        lib.canonical_matmul_id.argtypes = [ctypes.c_int, u32, u32, u32, u32, u32, ctypes.c_uint64,
                                            ctypes.c_int, P, P, P, P]
        lib.canonical_matmul_id_threads.argtypes = [ctypes.c_int, u32, u32, u32, u32, u32, ctypes.c_uint64,
                                                    ctypes.c_int, P, P, P, P, ctypes.c_int]
        _canon = lib
    return _canon


def host_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def canonical_matmul_id(wl, wbytes: np.ndarray, x: np.ndarray, ids: np.ndarray, threads: int = 1) -> np.ndarray:
    lib = _canonical_lib()
    wb = np.ascontiguousarray(wbytes, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    y = np.empty((wl.m * wl.top_k, wl.n), dtype=np.float32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    if threads > 1:
        rc = lib.canonical_matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride,
                                             wl.layout, p(wb), p(x), p(ids), p(y), threads)
        assert rc == 0, "canonical evaluation: out of host memory"
    else:
        lib.canonical_matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride,
                                wl.layout, p(wb), p(x), p(ids), p(y))
    return y


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def ids_to_dev(ids: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.uint32).view(np.int32)).to(device)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)
