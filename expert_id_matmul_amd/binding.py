"""ctypes binding of libeidm.so (include/eidm.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch CUDA tensors (device memory); the stream is the
caller's current torch stream unless one is given.  The binding refuses to
run when the library is missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeidm.so")

F32, F16, BF16 = 0, 1, 2
SHARED_PER_TOKEN, SLOTTED = 0, 1
DISTINCT_PER_TOKEN, MAY_REPEAT = 0, 1
AUTO, DIRECT, GROUPED = 0, 1, 2
ARITH_F32, ARITH_SPLIT16 = 0, 1
OK, E_INVALID, E_UNSUPPORTED, E_SIZE, E_ALIGN, E_DEVICE, E_IDS = 0, -1, -2, -3, -4, -5, -6

EXPORTS = ["eidm_abi_version", "eidm_last_error", "eidm_query", "eidm_route_topk", "eidm_map",
           "eidm_map_scratch_bytes", "eidm_matmul_id", "eidm_combine", "eidm_moe_forward",
           "eidm_validate_ids", "eidm_plan_create", "eidm_plan_destroy", "eidm_plan_freeze",
           "eidm_plan_route", "eidm_calibration_workspace_bytes", "eidm_calibrate",
           "eidm_matmul_id_planned", "eidm_moe_ffn_scratch_bytes", "eidm_moe_ffn", "eidm_matmul_id_noalloc",
           "eidm_last_dispatch", "eidm_plan_set_limits"]

# eidm_kernel (include/eidm.h): kernels a call can launch
KERNELS = {1: "route", 2: "map_one_pass", 3: "map_histogram", 4: "map_scatter", 5: "direct",
           6: "grouped_16x16", 7: "grouped_stream", 8: "grouped_job", 9: "combine",
           10: "fused_decode", 11: "silu_mul", 12: "validate", 13: "proof", 14: "split_x",
           15: "direct_split16", 16: "grouped_split16", 17: "map_split_x"}
MAX_RECORDED_LAUNCHES = 16


class Shape(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("weight_dtype", ctypes.c_int32),
                ("m", ctypes.c_uint32), ("n", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("top_k", ctypes.c_uint32), ("n_experts", ctypes.c_uint32),
                ("arith", ctypes.c_int32), ("expert_stride_bytes", ctypes.c_uint64),
                ("input_layout", ctypes.c_int32), ("id_multiplicity", ctypes.c_int32)]


class Requirements(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("route", ctypes.c_int32),
                ("required_weight_bytes", ctypes.c_uint64), ("input_elements", ctypes.c_uint64),
                ("ids_elements", ctypes.c_uint64), ("output_elements", ctypes.c_uint64),
                ("scratch_bytes", ctypes.c_uint64), ("grouped_legal", ctypes.c_int32),
                ("reserved0", ctypes.c_int32)]


class FfnShape(ctypes.Structure):
    """eidm_ffn_shape (include/eidm.h)."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("weight_dtype", ctypes.c_int32),
                ("m", ctypes.c_uint32), ("hidden", ctypes.c_uint32), ("inter", ctypes.c_uint32),
                ("top_k", ctypes.c_uint32), ("n_experts", ctypes.c_uint32), ("reserved0", ctypes.c_uint32),
                ("gate_up_stride_bytes", ctypes.c_uint64), ("down_stride_bytes", ctypes.c_uint64)]


def ffn_shape_of(fw) -> FfnShape:
    """The eidm_ffn_shape of a workloads.FfnWorkload."""
    size = 4 if fw.dtype == 0 else 2
    s = FfnShape()
    s.struct_size = ctypes.sizeof(FfnShape)
    s.weight_dtype, s.m, s.hidden, s.inter = fw.dtype, fw.m, fw.hidden, fw.inter
    s.top_k, s.n_experts = fw.top_k, fw.n_experts
    s.gate_up_stride_bytes = fw.inter * fw.hidden * size
    s.down_stride_bytes = fw.hidden * fw.inter * size
    return s


class Calibration(ctypes.Structure):
    """eidm_calibration (include/eidm.h)."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("route", ctypes.c_int32),
                ("grouped_legal", ctypes.c_int32), ("bit_identical", ctypes.c_int32),
                ("reason", ctypes.c_int32), ("submissions", ctypes.c_uint32)] + [
        (name, ctypes.c_double * 2) for name in (
            "direct_wall_p25", "direct_wall_median", "direct_wall_p75", "direct_gpu_median",
            "grouped_wall_p25", "grouped_wall_median", "grouped_wall_p75", "grouped_gpu_median")]

    def as_dict(self) -> dict:
        return {name: (list(getattr(self, name)) if isinstance(getattr(self, name), ctypes.Array)
                       else getattr(self, name)) for name, _ in self._fields_}


CAL_REASONS = ["grouped wins", "grouped not legal", "grouped failed", "not bit identical",
               "wall median", "wall quartiles", "gpu median", "budget"]
CAL_BUDGET = 7
GATE_SUBMISSIONS = 27  # host waits of one complete calibration gate


class CalibrationLimits(ctypes.Structure):
    """eidm_calibration_limits (include/eidm.h)."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("max_cases", ctypes.c_uint32),
                ("max_submissions", ctypes.c_uint32), ("reserved0", ctypes.c_uint32),
                ("max_elapsed_ms", ctypes.c_uint64)]


class Launch(ctypes.Structure):
    """eidm_launch (include/eidm.h)."""
    _fields_ = [("kernel", ctypes.c_int32), ("grid", ctypes.c_uint32), ("block", ctypes.c_uint32),
                ("lds_bytes", ctypes.c_uint32)]


class Dispatch(ctypes.Structure):
    """eidm_dispatch (include/eidm.h)."""
    _fields_ = [("struct_size", ctypes.c_uint32), ("route", ctypes.c_int32),
                ("dispatch_count", ctypes.c_uint32), ("recorded", ctypes.c_uint32),
                ("launches", Launch * MAX_RECORDED_LAUNCHES)]

    def kernels(self) -> list[str]:
        return [KERNELS.get(self.launches[i].kernel, "?") for i in range(self.recorded)]


class EidmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"eidm error {code}: {message}")
        self.code = code


def make_shape(dtype: int, m: int, n: int, k: int, top_k: int, n_experts: int, stride: int,
               layout: int = SHARED_PER_TOKEN, multiplicity: int = DISTINCT_PER_TOKEN,
               arith: int = ARITH_F32) -> Shape:
    return Shape(ctypes.sizeof(Shape), dtype, m, n, k, top_k, n_experts, arith, stride, layout,
                 multiplicity)


def shape_of(wl) -> Shape:
    """Shape key of a workloads.Workload."""
    return make_shape(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout,
                      wl.multiplicity, wl.arith)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need(name: str, t, elements: int, itemsize: int = 4, optional: bool = False) -> None:
    """Refuse host tensors and tensors smaller than the call will touch."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return  # a raw device address: the caller vouches for it
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _nbytes(t) < elements * itemsize:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, the call needs {elements * itemsize}")


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


class Library:
    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first (python -m expert_id_matmul_amd.build)")
        self.path = path
        self.lib = ctypes.CDLL(path)
        L = self.lib
        P, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
        L.eidm_abi_version.restype = i32
        L.eidm_abi_version.argtypes = []
        L.eidm_last_error.restype = ctypes.c_char_p
        L.eidm_last_error.argtypes = []
        L.eidm_query.restype = i32
        L.eidm_query.argtypes = [ctypes.POINTER(Shape), i32, ctypes.POINTER(Requirements)]
        L.eidm_route_topk.restype = i32
        L.eidm_route_topk.argtypes = [P, P, u32, u32, u32, i32, P, P, P]
        L.eidm_map.restype = i32
        L.eidm_map.argtypes = [P, u32, u32, u32, P, P, P, P, u64, P]
        L.eidm_map_scratch_bytes.restype = u64
        L.eidm_map_scratch_bytes.argtypes = [u32, u32, u32]
        L.eidm_matmul_id.restype = i32
        L.eidm_matmul_id.argtypes = [ctypes.POINTER(Shape), i32, P, u64, P, P, P, P, u64, P,
                                     ctypes.POINTER(ctypes.c_int)]
        L.eidm_matmul_id_noalloc.restype = i32
        L.eidm_matmul_id_noalloc.argtypes = [ctypes.POINTER(Shape), i32, P, u64, P, P, P, P,
                                             ctypes.POINTER(ctypes.c_int)]
        L.eidm_combine.restype = i32
        L.eidm_combine.argtypes = [u32, u32, u32, P, P, P, P]
        L.eidm_validate_ids.restype = i32
        L.eidm_validate_ids.argtypes = [P, u32, u32, u32, i32, ctypes.POINTER(ctypes.c_int32), P]
        L.eidm_plan_create.restype = P
        L.eidm_plan_create.argtypes = []
        L.eidm_plan_destroy.restype = None
        L.eidm_plan_destroy.argtypes = [P]
        L.eidm_plan_freeze.restype = i32
        L.eidm_plan_freeze.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
        L.eidm_plan_set_limits.restype = i32
        L.eidm_plan_set_limits.argtypes = [P, ctypes.POINTER(CalibrationLimits)]
        L.eidm_last_dispatch.restype = i32
        L.eidm_last_dispatch.argtypes = [ctypes.POINTER(Dispatch)]
        L.eidm_plan_route.restype = i32
        L.eidm_plan_route.argtypes = [P, ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_int)]
        L.eidm_calibration_workspace_bytes.restype = u64
        L.eidm_calibration_workspace_bytes.argtypes = [ctypes.POINTER(Shape)]
        L.eidm_calibrate.restype = i32
        L.eidm_calibrate.argtypes = [P, ctypes.POINTER(Shape), P, u64, P, u64, P, ctypes.POINTER(Calibration)]
        L.eidm_matmul_id_planned.restype = i32
        L.eidm_matmul_id_planned.argtypes = [P, ctypes.POINTER(Shape), P, u64, P, P, P, P, u64, P,
                                             ctypes.POINTER(ctypes.c_int)]
        L.eidm_moe_ffn_scratch_bytes.restype = u64
        L.eidm_moe_ffn_scratch_bytes.argtypes = [ctypes.POINTER(FfnShape)]
        L.eidm_moe_ffn.restype = i32
        L.eidm_moe_ffn.argtypes = [ctypes.POINTER(FfnShape), i32, P, P, u64, P, u64, P, P, P, i32, P, P, P, P,
                                   u64, P, ctypes.POINTER(ctypes.c_int)]
        L.eidm_moe_forward.restype = i32
        L.eidm_moe_forward.argtypes = [ctypes.POINTER(Shape), i32, P, u64, P, P, P, i32, P, P, P, P,
                                       P, u64, P, ctypes.POINTER(ctypes.c_int)]

    # ------------------------------------------------------------------ helpers
    def _check(self, rc: int) -> None:
        if rc != OK:
            raise EidmError(rc, self.lib.eidm_last_error().decode())

    def last_error(self) -> str:
        return self.lib.eidm_last_error().decode()

    def abi_version(self) -> int:
        return self.lib.eidm_abi_version()

    def last_dispatch(self) -> Dispatch:
        """The dispatch receipt of this thread's last library call."""
        d = Dispatch()
        d.struct_size = ctypes.sizeof(Dispatch)
        self._check(self.lib.eidm_last_dispatch(ctypes.byref(d)))
        return d

    def _check_matmul_buffers(self, shape, route, weights, weight_bytes, input, ids, output,
                              scratch) -> None:
        req = self.query(shape, route)
        _need("weights", weights, weight_bytes, 1)
        _need("input", input, req.input_elements)
        _need("ids", ids, req.ids_elements)
        _need("output", output, req.output_elements)
        if scratch is not None:
            _need("scratch", scratch, 0, 1)

    # ------------------------------------------------------------------ ABI calls
    def query(self, shape: Shape, route: int = AUTO) -> Requirements:
        req = Requirements()
        req.struct_size = ctypes.sizeof(Requirements)
        self._check(self.lib.eidm_query(ctypes.byref(shape), route, ctypes.byref(req)))
        return req

    def route_topk(self, logits, bias, top_k: int, ids, gates, renormalize: bool = True,
                   stream=None) -> None:
        m, n_experts = logits.shape
        _need("logits", logits, m * n_experts)
        _need("bias", bias, n_experts, optional=True)
        _need("ids", ids, m * top_k)
        _need("gates", gates, m * top_k, optional=True)
        self._check(self.lib.eidm_route_topk(_ptr(logits), _ptr(bias), m, n_experts, top_k,
                                             int(renormalize), _ptr(ids), _ptr(gates),
                                             _stream(stream)))

    def map_scratch_bytes(self, m: int, top_k: int, n_experts: int) -> int:
        return int(self.lib.eidm_map_scratch_bytes(m, top_k, n_experts))

    def map(self, ids, n_experts: int, counts, offsets, rows, scratch, stream=None) -> None:
        m, top_k = ids.shape
        _need("ids", ids, m * top_k)
        _need("counts", counts, n_experts + 1)
        _need("offsets", offsets, n_experts + 2)
        _need("rows", rows, m * top_k)
        _need("scratch", scratch, self.map_scratch_bytes(m, top_k, n_experts), 1)
        nbytes = _nbytes(scratch)
        self._check(self.lib.eidm_map(_ptr(ids), m, top_k, n_experts, _ptr(counts), _ptr(offsets),
                                      _ptr(rows), _ptr(scratch), nbytes, _stream(stream)))

    def matmul_id(self, shape: Shape, route: int, weights, input, ids, output, scratch=None,
                  weight_bytes: int | None = None, stream=None) -> int:
        if weight_bytes is None:
            weight_bytes = _nbytes(weights)
        self._check_matmul_buffers(shape, route, weights, weight_bytes, input, ids, output, scratch)
        sbytes = _nbytes(scratch) if scratch is not None else 0
        taken = ctypes.c_int(-1)
        self._check(self.lib.eidm_matmul_id(ctypes.byref(shape), route, _ptr(weights), weight_bytes,
                                            _ptr(input), _ptr(ids), _ptr(output), _ptr(scratch),
                                            sbytes, _stream(stream), ctypes.byref(taken)))
        return taken.value

    def matmul_id_noalloc(self, shape: Shape, route: int, weights, input, ids, output,
                          weight_bytes: int | None = None, stream=None) -> int:
        """eidm_matmul_id with the library's static map array (no scratch)."""
        if weight_bytes is None:
            weight_bytes = _nbytes(weights)
        self._check_matmul_buffers(shape, DIRECT, weights, weight_bytes, input, ids, output, None)
        taken = ctypes.c_int(-1)
        self._check(self.lib.eidm_matmul_id_noalloc(ctypes.byref(shape), route, _ptr(weights), weight_bytes,
                                                    _ptr(input), _ptr(ids), _ptr(output), _stream(stream),
                                                    ctypes.byref(taken)))
        return taken.value

    def combine(self, y, gates, out, stream=None) -> None:
        m, top_k = gates.shape
        n = y.shape[-1]
        _need("y", y, m * top_k * n)
        _need("gates", gates, m * top_k)
        _need("out", out, m * n)
        self._check(self.lib.eidm_combine(m, top_k, n, _ptr(y), _ptr(gates), _ptr(out),
                                          _stream(stream)))

    def moe_forward(self, shape: Shape, route: int, weights, input, logits, bias, ids, gates, y,
                    out, scratch=None, renormalize: bool = True, weight_bytes: int | None = None,
                    stream=None) -> int:
        if weight_bytes is None:
            weight_bytes = _nbytes(weights)
        self._check_matmul_buffers(shape, route, weights, weight_bytes, input, ids, y, scratch)
        _need("logits", logits, shape.m * shape.n_experts)
        _need("bias", bias, shape.n_experts, optional=True)
        _need("gates", gates, shape.m * shape.top_k)
        _need("out", out, shape.m * shape.n)
        sbytes = _nbytes(scratch) if scratch is not None else 0
        taken = ctypes.c_int(-1)
        self._check(self.lib.eidm_moe_forward(ctypes.byref(shape), route, _ptr(weights),
                                              weight_bytes, _ptr(input), _ptr(logits), _ptr(bias),
                                              int(renormalize), _ptr(ids), _ptr(gates), _ptr(y),
                                              _ptr(out), _ptr(scratch), sbytes, _stream(stream),
                                              ctypes.byref(taken)))
        return taken.value

    def validate_ids(self, ids, n_experts: int, multiplicity: int = 0, stream=None) -> int:
        """The smallest bad routed index of ids [m, top_k], or -1 (synchronous)."""
        m, top_k = ids.shape
        _need("ids", ids, m * top_k)
        bad = ctypes.c_int32(-2)
        rc = self.lib.eidm_validate_ids(_ptr(ids), m, top_k, n_experts, multiplicity, ctypes.byref(bad),
                                        _stream(stream))
        if rc not in (OK, E_IDS):
            self._check(rc)
        return bad.value

    def moe_ffn_scratch_bytes(self, shape: FfnShape) -> int:
        return self.lib.eidm_moe_ffn_scratch_bytes(ctypes.byref(shape))

    def moe_ffn(self, shape: FfnShape, route: int, w_gate, w_up, w_down, x, logits, bias, ids, gates, out,
                scratch, renormalize: bool = True, stream=None) -> int:
        m, hidden, inter, top_k, E = shape.m, shape.hidden, shape.inter, shape.top_k, shape.n_experts
        gu_bytes = min(_nbytes(w_gate), _nbytes(w_up))
        _need("w_gate", w_gate, gu_bytes, 1)
        _need("w_up", w_up, gu_bytes, 1)
        _need("w_down", w_down, _nbytes(w_down), 1)
        _need("x", x, m * hidden)
        _need("logits", logits, m * E)
        _need("bias", bias, E, optional=True)
        _need("ids", ids, m * top_k)
        _need("gates", gates, m * top_k)
        _need("out", out, m * hidden)
        _need("scratch", scratch, self.moe_ffn_scratch_bytes(shape), 1)
        taken = ctypes.c_int(-1)
        self._check(self.lib.eidm_moe_ffn(ctypes.byref(shape), route, _ptr(w_gate), _ptr(w_up), gu_bytes,
                                          _ptr(w_down), _nbytes(w_down), _ptr(x), _ptr(logits), _ptr(bias),
                                          int(renormalize), _ptr(ids), _ptr(gates), _ptr(out), _ptr(scratch),
                                          _nbytes(scratch), _stream(stream), ctypes.byref(taken)))
        return taken.value


class Plan:
    """A route plan (eidm_plan): activation-time calibration of exact shapes,
    then lookups; the plan is destroyed with this object."""

    def __init__(self, lib: Library):
        self.lib = lib
        self.handle = lib.lib.eidm_plan_create()
        if not self.handle:
            raise MemoryError("eidm_plan_create")

    def __del__(self):
        if getattr(self, "handle", None):
            self.lib.lib.eidm_plan_destroy(ctypes.c_void_p(self.handle))
            self.handle = None

    def workspace_bytes(self, shape: Shape) -> int:
        return self.lib.lib.eidm_calibration_workspace_bytes(ctypes.byref(shape))

    def calibrate(self, shape: Shape, weights, workspace, weight_bytes: int | None = None,
                  stream=None) -> Calibration:
        if weight_bytes is None:
            weight_bytes = _nbytes(weights)
        _need("weights", weights, weight_bytes, 1)
        _need("workspace", workspace, self.workspace_bytes(shape), 1)
        rec = Calibration()
        rec.struct_size = ctypes.sizeof(Calibration)
        self.lib._check(self.lib.lib.eidm_calibrate(ctypes.c_void_p(self.handle), ctypes.byref(shape),
                                                    _ptr(weights), weight_bytes, _ptr(workspace),
                                                    _nbytes(workspace), _stream(stream), ctypes.byref(rec)))
        return rec

    def set_limits(self, max_elapsed_ms: int = 15000, max_cases: int = 256,
                   max_submissions: int = 6145) -> None:
        lim = CalibrationLimits(ctypes.sizeof(CalibrationLimits), max_cases, max_submissions, 0,
                                max_elapsed_ms)
        self.lib._check(self.lib.lib.eidm_plan_set_limits(ctypes.c_void_p(self.handle), ctypes.byref(lim)))

    def freeze(self) -> int:
        """Freeze the plan; returns how many Grouped entries the deadline turned into Direct."""
        n = ctypes.c_uint32(0)
        self.lib._check(self.lib.lib.eidm_plan_freeze(ctypes.c_void_p(self.handle), ctypes.byref(n)))
        return n.value

    def route(self, shape: Shape) -> int:
        r = ctypes.c_int(-1)
        self.lib._check(self.lib.lib.eidm_plan_route(ctypes.c_void_p(self.handle), ctypes.byref(shape),
                                                     ctypes.byref(r)))
        return r.value

    def matmul_id(self, shape: Shape, weights, input, ids, output, scratch=None,
                  weight_bytes: int | None = None, stream=None) -> int:
        if weight_bytes is None:
            weight_bytes = _nbytes(weights)
        route = self.route(shape)
        self.lib._check_matmul_buffers(shape, route, weights, weight_bytes, input, ids, output, scratch)
        sbytes = _nbytes(scratch) if scratch is not None else 0
        taken = ctypes.c_int(-1)
        self.lib._check(self.lib.lib.eidm_matmul_id_planned(
            ctypes.c_void_p(self.handle), ctypes.byref(shape), _ptr(weights), weight_bytes, _ptr(input),
            _ptr(ids), _ptr(output), _ptr(scratch), sbytes, _stream(stream), ctypes.byref(taken)))
        return taken.value


_LIB: Library | None = None


def load(path: str = LIB_PATH) -> Library:
    global _LIB
    if _LIB is None or _LIB.path != path:
        _LIB = Library(path)
    return _LIB
