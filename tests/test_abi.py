"""The C-ABI boundary on the CPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host before any launch
(so none of these tests touches a GPU)."""
import ctypes
import os
import re

import pytest

from expert_id_matmul_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eidm.h")

# never dereferenced: every call below fails validation first
FAKE = 0x7F0000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eidm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_what_the_binding_uses():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib.lib, name), name
    assert lib.abi_version() == 2


def test_struct_sizes_match_the_header_layout():
    assert ctypes.sizeof(B.Shape) == 48
    assert ctypes.sizeof(B.Requirements) == 56
    assert ctypes.sizeof(B.Launch) == 16
    assert ctypes.sizeof(B.Dispatch) == 16 + 16 * B.MAX_RECORDED_LAUNCHES
    assert ctypes.sizeof(B.CalibrationLimits) == 24
    assert ctypes.sizeof(B.Calibration) == 24 + 8 * 2 * 8


def test_query_reports_the_pages_weight_extent_and_sizes(lib):
    # mlx-native dense_matmul_id_auto.rs, A-B-A test: n=5, k=7, 4 experts,
    # stride 152 -> a 596-byte weight buffer
    s = B.make_shape(B.F32, 3, 5, 7, 3, 4, 152)
    r = lib.query(s, B.DIRECT)
    assert r.required_weight_bytes == 596
    assert r.input_elements == 3 * 7 and r.ids_elements == 9 and r.output_elements == 9 * 5
    assert r.route == B.DIRECT and r.scratch_bytes == 0 and r.grouped_legal == 1
    g = lib.query(s, B.GROUPED)
    assert g.route == B.GROUPED and g.scratch_bytes > 0
    slotted = lib.query(B.make_shape(B.F32, 3, 5, 7, 3, 4, 152, B.SLOTTED), B.DIRECT)
    assert slotted.input_elements == 9 * 7


def test_query_auto_picks_direct_for_decode_and_grouped_for_prefill(lib):
    dec = B.make_shape(B.BF16, 1, 1536, 4096, 8, 256, 1536 * 4096 * 2)
    assert lib.query(dec, B.AUTO).route == B.DIRECT
    pre = B.make_shape(B.BF16, 512, 768, 2048, 8, 128, 768 * 2048 * 2)
    assert lib.query(pre, B.AUTO).route == B.GROUPED


@pytest.mark.parametrize("field,value,code", [
    ("m", 0, B.E_INVALID), ("n", 0, B.E_INVALID), ("k", 0, B.E_INVALID),
    ("top_k", 0, B.E_INVALID), ("n_experts", 0, B.E_INVALID),
    ("weight_dtype", 7, B.E_INVALID), ("input_layout", 2, B.E_INVALID),
    ("id_multiplicity", 5, B.E_INVALID), ("arith", 2, B.E_INVALID),
    ("struct_size", 40, B.E_INVALID), ("top_k", 5, B.E_INVALID),  # 5 distinct of 4
    ("expert_stride_bytes", 139, B.E_ALIGN),  # not a multiple of 4
    ("expert_stride_bytes", 136, B.E_INVALID),  # shorter than one expert (140 B)
    ("n_experts", 4096, B.E_UNSUPPORTED),
    ("m", 2 ** 31, B.E_UNSUPPORTED),
])
def test_query_rejects_bad_shapes(lib, field, value, code):
    s = B.make_shape(B.F32, 3, 5, 7, 3, 4, 152)
    setattr(s, field, value)
    with pytest.raises(B.EidmError) as ei:
        lib.query(s, B.DIRECT)
    assert ei.value.code == code, lib.last_error()
    assert lib.last_error()


def test_query_rejects_overflowing_extents(lib):
    s = B.make_shape(B.F32, 1, 65536, 65536, 1, 2000, 2 ** 62)
    with pytest.raises(B.EidmError) as ei:
        lib.query(s, B.DIRECT)
    assert ei.value.code == B.E_INVALID


def test_may_repeat_allows_top_k_above_n_experts(lib):
    s = B.make_shape(B.F32, 3, 5, 7, 6, 4, 152, B.SHARED_PER_TOKEN, B.MAY_REPEAT)
    assert lib.query(s, B.GROUPED).grouped_legal == 1


def test_unknown_route_is_rejected(lib):
    with pytest.raises(B.EidmError):
        lib.query(B.make_shape(B.F32, 3, 5, 7, 3, 4, 152), 9)


def _matmul(lib, shape, route=B.DIRECT, weights=FAKE, wbytes=596, inp=FAKE, ids=FAKE,
            out=FAKE, scratch=0, sbytes=0):
    taken = ctypes.c_int(-1)
    rc = lib.lib.eidm_matmul_id(ctypes.byref(shape), route, ctypes.c_void_p(weights), wbytes,
                                ctypes.c_void_p(inp), ctypes.c_void_p(ids), ctypes.c_void_p(out),
                                ctypes.c_void_p(scratch), sbytes, None, ctypes.byref(taken))
    return rc, taken.value


def test_matmul_rejects_before_launch(lib):
    s = B.make_shape(B.F32, 3, 5, 7, 3, 4, 152)
    # short weight extent (595 < 596)
    assert _matmul(lib, s, wbytes=595) == (B.E_SIZE, -1)
    # weights misaligned for f32
    assert _matmul(lib, s, weights=FAKE + 2)[0] == B.E_ALIGN
    # null pointers
    assert _matmul(lib, s, weights=0)[0] == B.E_INVALID
    assert _matmul(lib, s, out=0)[0] == B.E_INVALID
    assert _matmul(lib, s, ids=FAKE + 1)[0] == B.E_ALIGN
    # grouped without scratch / with too little / misaligned
    assert _matmul(lib, s, route=B.GROUPED)[0] == B.E_SIZE
    assert _matmul(lib, s, route=B.GROUPED, scratch=FAKE, sbytes=8)[0] == B.E_SIZE
    need = lib.query(s, B.GROUPED).scratch_bytes
    assert _matmul(lib, s, route=B.GROUPED, scratch=FAKE + 64, sbytes=need)[0] == B.E_ALIGN
    # bf16 weights need 2-byte alignment only
    sb = B.make_shape(B.BF16, 9, 11, 37, 6, 8, 832)
    assert _matmul(lib, sb, weights=FAKE + 3, wbytes=10 ** 6)[0] == B.E_ALIGN


def test_noalloc_rejects_a_map_beyond_its_static_array_before_launch(lib):
    # 400000 tokens x top-8: the id -> row map alone needs about 12.8 MB, above
    # the 8 MiB array; the call fails on the host (no pointer is touched)
    s = B.make_shape(B.BF16, 400000, 64, 256, 8, 16, 64 * 256 * 2)
    assert lib.query(s, B.GROUPED).scratch_bytes > 8 << 20
    taken = ctypes.c_int(-1)
    rc = lib.lib.eidm_matmul_id_noalloc(ctypes.byref(s), B.GROUPED, None, 0, None, None, None, None,
                                        ctypes.byref(taken))
    assert rc == B.E_SIZE and "static array" in lib.last_error()
    assert taken.value == -1
    # a bad shape is rejected the same way as by eidm_matmul_id
    bad = B.make_shape(B.BF16, 0, 64, 256, 8, 16, 64 * 256 * 2)
    assert lib.lib.eidm_matmul_id_noalloc(ctypes.byref(bad), B.AUTO, None, 0, None, None, None, None,
                                          None) == B.E_INVALID


def test_route_map_combine_reject_bad_arguments(lib):
    L = lib.lib
    P = ctypes.c_void_p
    assert L.eidm_route_topk(P(FAKE), None, 4, 8, 9, 1, P(FAKE), None, None) == B.E_INVALID
    assert L.eidm_route_topk(P(FAKE), None, 0, 8, 2, 1, P(FAKE), None, None) == B.E_INVALID
    assert L.eidm_route_topk(None, None, 4, 8, 2, 1, P(FAKE), None, None) == B.E_INVALID
    assert L.eidm_route_topk(P(FAKE), None, 4, 4096, 2, 1, P(FAKE), None, None) == B.E_UNSUPPORTED
    assert L.eidm_route_topk(P(FAKE + 2), None, 4, 8, 2, 1, P(FAKE), None, None) == B.E_ALIGN
    assert L.eidm_route_topk(P(FAKE), None, 4, 128, 65, 1, P(FAKE), None, None) == B.E_UNSUPPORTED
    assert L.eidm_combine(0, 2, 8, P(FAKE), P(FAKE), P(FAKE), None) == B.E_INVALID
    assert L.eidm_combine(2, 2, 8, None, P(FAKE), P(FAKE), None) == B.E_INVALID
    assert L.eidm_combine(2, 2, 8, P(FAKE + 1), P(FAKE), P(FAKE), None) == B.E_ALIGN
    need = lib.map_scratch_bytes(10, 2, 8)
    assert need == 9 * 4  # one block of rows, n_experts + 1 counters
    assert L.eidm_map(P(FAKE), 10, 2, 8, P(FAKE), P(FAKE), P(FAKE), P(FAKE), need - 4, None) == B.E_SIZE
    assert L.eidm_map(P(FAKE), 10, 2, 0, P(FAKE), P(FAKE), P(FAKE), P(FAKE), need, None) == B.E_INVALID


def test_moe_forward_requires_distinct_ids(lib):
    s = B.make_shape(B.F32, 3, 5, 7, 3, 4, 152, B.SHARED_PER_TOKEN, B.MAY_REPEAT)
    P = ctypes.c_void_p
    rc = lib.lib.eidm_moe_forward(ctypes.byref(s), B.DIRECT, P(FAKE), 596, P(FAKE), P(FAKE), None, 1,
                                  P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, 0, None, None)
    assert rc == B.E_INVALID


def test_validate_ids_rejects_bad_arguments_before_launch(lib):
    L = lib.lib
    P = ctypes.c_void_p
    bad = ctypes.c_int32(7)
    assert L.eidm_validate_ids(None, 4, 2, 8, 0, ctypes.byref(bad), None) == B.E_INVALID
    assert L.eidm_validate_ids(P(FAKE), 4, 2, 8, 0, None, None) == B.E_INVALID
    assert L.eidm_validate_ids(P(FAKE), 0, 2, 8, 0, ctypes.byref(bad), None) == B.E_INVALID
    assert L.eidm_validate_ids(P(FAKE), 4, 2, 8, 5, ctypes.byref(bad), None) == B.E_INVALID
    assert L.eidm_validate_ids(P(FAKE + 2), 4, 2, 8, 0, ctypes.byref(bad), None) == B.E_ALIGN
    assert L.eidm_validate_ids(P(FAKE), 1 << 30, 4, 8, 0, ctypes.byref(bad), None) == B.E_UNSUPPORTED
    assert bad.value == 7  # untouched on failure


def test_calibration_struct_and_plan_rules_on_the_host(lib):
    """Plan lifecycle and every argument check of the calibration entry points
    run on the host before any device work."""
    assert ctypes.sizeof(B.Calibration) == 152
    L = lib.lib
    P = ctypes.c_void_p
    plan = P(L.eidm_plan_create())
    assert plan.value
    s = B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2, B.SHARED_PER_TOKEN, B.DISTINCT_PER_TOKEN)
    route = ctypes.c_int(-1)
    assert L.eidm_plan_route(plan, ctypes.byref(s), ctypes.byref(route)) == B.E_UNSUPPORTED
    assert L.eidm_matmul_id_planned(plan, ctypes.byref(s), P(FAKE), 16 * 128 * 256 * 2, P(FAKE), P(FAKE),
                                    P(FAKE), None, 0, None, None) == B.E_UNSUPPORTED
    need = L.eidm_calibration_workspace_bytes(ctypes.byref(s))
    assert need > 64 * 256 * 4 + 2 * (64 * 4 * 128 + 16) * 4  # activations, two outputs with guards
    rec = B.Calibration()
    rec.struct_size = ctypes.sizeof(B.Calibration)
    wb = 16 * 128 * 256 * 2
    assert L.eidm_calibrate(None, ctypes.byref(s), P(FAKE), wb, P(FAKE), need, None, ctypes.byref(rec)) == B.E_INVALID
    assert L.eidm_calibrate(plan, ctypes.byref(s), P(FAKE), wb, P(FAKE), need - 1, None,
                            ctypes.byref(rec)) == B.E_SIZE
    assert L.eidm_calibrate(plan, ctypes.byref(s), P(FAKE), wb, P(FAKE + 64), need, None,
                            ctypes.byref(rec)) == B.E_ALIGN
    rec.struct_size = 8
    assert L.eidm_calibrate(plan, ctypes.byref(s), P(FAKE), wb, P(FAKE), need, None, ctypes.byref(rec)) == B.E_INVALID
    rec.struct_size = ctypes.sizeof(B.Calibration)
    bad = B.make_shape(B.BF16, 0, 128, 256, 4, 16, 128 * 256 * 2, B.SHARED_PER_TOKEN, B.DISTINCT_PER_TOKEN)
    assert L.eidm_calibration_workspace_bytes(ctypes.byref(bad)) == 0
    assert L.eidm_plan_freeze(plan, None) == B.OK
    assert L.eidm_calibrate(plan, ctypes.byref(s), P(FAKE), wb, P(FAKE), need, None, ctypes.byref(rec)) == B.E_INVALID
    L.eidm_plan_destroy(plan)


def test_moe_ffn_rejects_bad_arguments_before_launch(lib):
    L = lib.lib
    P = ctypes.c_void_p
    s = B.FfnShape()
    s.struct_size = ctypes.sizeof(B.FfnShape)
    s.weight_dtype, s.m, s.hidden, s.inter, s.top_k, s.n_experts = B.BF16, 8, 64, 32, 2, 4
    s.gate_up_stride_bytes = 32 * 64 * 2
    s.down_stride_bytes = 64 * 32 * 2
    assert ctypes.sizeof(B.FfnShape) == 48
    need = L.eidm_moe_ffn_scratch_bytes(ctypes.byref(s))
    assert need >= (2 * 8 * 2 * 32 + 8 * 2 * 64) * 4
    wb = 4 * 32 * 64 * 2
    args = lambda **kw: [ctypes.byref(kw.get("shape", s)), B.AUTO, P(FAKE), P(FAKE), kw.get("gub", wb), P(FAKE),
                         kw.get("db", wb), P(FAKE), P(FAKE), None, 1, P(FAKE), P(FAKE), P(FAKE),
                         kw.get("scratch", P(FAKE)), kw.get("sb", need), None, None]
    assert L.eidm_moe_ffn(*args(sb=need - 1)) == B.E_SIZE
    assert L.eidm_moe_ffn(*args(gub=wb - 2)) == B.E_SIZE
    assert L.eidm_moe_ffn(*args(db=wb - 2)) == B.E_SIZE
    assert L.eidm_moe_ffn(*args(scratch=P(FAKE + 128))) == B.E_ALIGN
    assert L.eidm_moe_ffn(*args(scratch=None)) == B.E_INVALID
    bad = B.FfnShape.from_buffer_copy(s)
    bad.struct_size = 40
    assert L.eidm_moe_ffn(*args(shape=bad)) == B.E_INVALID
    assert L.eidm_moe_ffn_scratch_bytes(ctypes.byref(bad)) == 0
    bad = B.FfnShape.from_buffer_copy(s)
    bad.top_k = 5  # more distinct picks than experts
    assert L.eidm_moe_ffn(*args(shape=bad)) == B.E_INVALID
    bad = B.FfnShape.from_buffer_copy(s)
    bad.n_experts, bad.top_k = 4096, 65  # past the router's limits
    assert L.eidm_moe_ffn(*args(shape=bad, gub=4096 * 32 * 64 * 2, db=4096 * 32 * 64 * 2)) == B.E_UNSUPPORTED


def test_dispatch_receipt_rules_and_a_rejected_call_enqueues_nothing(lib):
    """eidm_last_dispatch (mlx-native dense_matmul_id_auto.rs: the primitive's
    receipt): a call rejected on the host reports no route and no launch."""
    L = lib.lib
    assert L.eidm_last_dispatch(None) == B.E_INVALID
    d = B.Dispatch()
    d.struct_size = 8
    assert L.eidm_last_dispatch(ctypes.byref(d)) == B.E_INVALID
    s = B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2)
    P = ctypes.c_void_p
    # NULL output: rejected before anything is enqueued
    assert L.eidm_matmul_id(ctypes.byref(s), B.DIRECT, P(FAKE), 16 * 128 * 256 * 2, P(FAKE), P(FAKE), None,
                            None, 0, None, None) == B.E_INVALID
    d = lib.last_dispatch()
    assert (d.route, d.dispatch_count, d.recorded) == (0, 0, 0)
    assert d.struct_size == ctypes.sizeof(B.Dispatch)


def _cal_args(lib, s):
    need = lib.lib.eidm_calibration_workspace_bytes(ctypes.byref(s))
    assert need > 0
    rec = B.Calibration()
    rec.struct_size = ctypes.sizeof(B.Calibration)
    wb = s.n_experts * s.expert_stride_bytes
    return need, rec, wb


def _calibrate_no_gpu(lib, plan, s):
    """eidm_calibrate on fake addresses: only paths that enqueue nothing may
    run here (the budget and case rules are decided before any GPU work)."""
    need, rec, wb = _cal_args(lib, s)
    P = ctypes.c_void_p
    rc = lib.lib.eidm_calibrate(plan, ctypes.byref(s), P(FAKE), wb, P(FAKE), need, None, ctypes.byref(rec))
    return rc, rec


def _limits(ms, cases, subs, size=None):
    lim = B.CalibrationLimits(ctypes.sizeof(B.CalibrationLimits) if size is None else size, cases, subs, 0, ms)
    return ctypes.byref(lim)


def test_calibration_limits_must_be_nonzero_and_precede_calibration(lib):
    """DenseMatmulIdCalibrationLimits: every limit nonzero; the limits are fixed
    once calibration has begun."""
    L = lib.lib
    plan = L.eidm_plan_create()
    try:
        assert L.eidm_plan_set_limits(None, _limits(1, 1, 1)) == B.E_INVALID
        assert L.eidm_plan_set_limits(plan, None) == B.E_INVALID
        assert L.eidm_plan_set_limits(plan, _limits(1, 1, 1, size=16)) == B.E_INVALID
        for ms, cases, subs in ((0, 1, 1), (1, 0, 1), (1, 1, 0)):
            assert L.eidm_plan_set_limits(plan, _limits(ms, cases, subs)) == B.E_INVALID
        assert "nonzero" in lib.last_error()
        assert L.eidm_plan_set_limits(plan, _limits(15000, 256, B.GATE_SUBMISSIONS - 1)) == B.OK
        s = B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2)
        rc, rec = _calibrate_no_gpu(lib, plan, s)
        assert rc == B.OK
        assert L.eidm_plan_set_limits(plan, _limits(15000, 256, 6145)) == B.E_INVALID
    finally:
        L.eidm_plan_destroy(plan)


def test_calibration_without_budget_for_a_complete_gate_takes_direct(lib):
    """fn calibrate_one_inner: a shape whose proofs and timing the remaining
    submissions cannot pay for in full takes Direct with no GPU work."""
    L = lib.lib
    plan = L.eidm_plan_create()
    try:
        assert L.eidm_plan_set_limits(plan, _limits(15000, 256, B.GATE_SUBMISSIONS - 1)) == B.OK
        s = B.make_shape(B.BF16, 512, 128, 256, 4, 16, 128 * 256 * 2)
        rc, rec = _calibrate_no_gpu(lib, plan, s)
        assert rc == B.OK
        assert (rec.route, rec.reason, rec.submissions) == (B.DIRECT, B.CAL_BUDGET, 0)
        assert rec.grouped_legal == 1 and rec.bit_identical == 0
        assert list(rec.grouped_wall_median) == [0.0, 0.0]
        route = ctypes.c_int(-1)
        assert L.eidm_plan_route(plan, ctypes.byref(s), ctypes.byref(route)) == B.OK
        assert route.value == B.DIRECT
        assert lib.last_dispatch().dispatch_count == 0
        n = ctypes.c_uint32(99)
        assert L.eidm_plan_freeze(plan, ctypes.byref(n)) == B.OK and n.value == 0
    finally:
        L.eidm_plan_destroy(plan)


def test_calibration_after_the_deadline_takes_direct(lib):
    """The budget check before any proof: past max_elapsed_ms a shape takes
    Direct; freezing after the deadline has no Grouped entry to downgrade."""
    import time
    L = lib.lib
    plan = L.eidm_plan_create()
    try:
        assert L.eidm_plan_set_limits(plan, _limits(1, 256, 6145)) == B.OK
        time.sleep(0.01)
        s = B.make_shape(B.F16, 300, 64, 128, 2, 8, 64 * 128 * 2)
        rc, rec = _calibrate_no_gpu(lib, plan, s)
        assert rc == B.OK
        assert (rec.route, rec.reason, rec.submissions) == (B.DIRECT, B.CAL_BUDGET, 0)
        n = ctypes.c_uint32(99)
        assert L.eidm_plan_freeze(plan, ctypes.byref(n)) == B.OK and n.value == 0
    finally:
        L.eidm_plan_destroy(plan)


def test_calibration_case_limit_fails_closed(lib):
    """validate_cases: more distinct shapes than max_cases is an error and
    stores nothing; the same shape again is no new case."""
    L = lib.lib
    plan = L.eidm_plan_create()
    try:
        assert L.eidm_plan_set_limits(plan, _limits(15000, 2, 1)) == B.OK
        a = B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2)
        b = B.make_shape(B.BF16, 65, 128, 256, 4, 16, 128 * 256 * 2)
        c = B.make_shape(B.BF16, 64, 136, 256, 4, 16, 136 * 256 * 2)
        for s in (a, a, b, a):
            rc, rec = _calibrate_no_gpu(lib, plan, s)
            assert rc == B.OK and rec.reason == B.CAL_BUDGET
        rc, rec = _calibrate_no_gpu(lib, plan, c)
        assert rc == B.E_INVALID
        assert "2 cases" in lib.last_error()
        route = ctypes.c_int(-1)
        assert L.eidm_plan_route(plan, ctypes.byref(c), ctypes.byref(route)) == B.E_UNSUPPORTED
    finally:
        L.eidm_plan_destroy(plan)


def test_split16_shape_rules_and_scratch(lib):
    """The split-16 arithmetic: 16-bit weights only, k a multiple of 8; both
    routes need scratch for the split activations (three 16-bit parts per
    input element), Grouped the map as well."""
    s = B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2, arith=B.ARITH_SPLIT16)
    d = lib.query(s, B.DIRECT)
    g = lib.query(s, B.GROUPED)
    # three 16-bit parts per element, rows padded to whole 128-k rounds, a 256-byte zero block
    split = (256 + 64 * 2 * 16 * 48 + 255) // 256 * 256
    assert d.scratch_bytes == split
    s0 = B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2)
    assert lib.query(s0, B.DIRECT).scratch_bytes == 0
    assert g.scratch_bytes == lib.query(s0, B.GROUPED).scratch_bytes + split
    slot = B.make_shape(B.F16, 64, 128, 256, 4, 16, 128 * 256 * 2, layout=B.SLOTTED, arith=B.ARITH_SPLIT16)
    assert lib.query(slot, B.DIRECT).scratch_bytes == (256 + 64 * 4 * 2 * 16 * 48 + 255) // 256 * 256
    ragged = B.make_shape(B.BF16, 3, 128, 264, 4, 16, 128 * 264 * 2, arith=B.ARITH_SPLIT16)
    assert lib.query(ragged, B.DIRECT).scratch_bytes == (256 + 3 * 3 * 16 * 48 + 255) // 256 * 256
    for bad, code in [(B.make_shape(B.F32, 64, 128, 256, 4, 16, 128 * 256 * 4, arith=B.ARITH_SPLIT16), B.E_UNSUPPORTED),
                      (B.make_shape(B.BF16, 64, 128, 252, 4, 16, 128 * 252 * 2, arith=B.ARITH_SPLIT16), B.E_UNSUPPORTED),
                      (B.make_shape(B.BF16, 64, 128, 256, 4, 16, 128 * 256 * 2, arith=7), B.E_INVALID)]:
        with pytest.raises(B.EidmError) as e:
            lib.query(bad, B.DIRECT)
        assert e.value.code == code


def test_split16_rejects_before_launch(lib):
    L = lib.lib
    P = ctypes.c_void_p
    s = B.make_shape(B.BF16, 8, 64, 128, 2, 4, 64 * 128 * 2, arith=B.ARITH_SPLIT16)
    wb = 4 * 64 * 128 * 2
    need = lib.query(s, B.DIRECT).scratch_bytes
    # Direct needs the split scratch too
    assert L.eidm_matmul_id(ctypes.byref(s), B.DIRECT, P(FAKE), wb, P(FAKE), P(FAKE), P(FAKE), None, 0, None,
                            None) == B.E_SIZE
    assert L.eidm_matmul_id(ctypes.byref(s), B.DIRECT, P(FAKE), wb, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                            need - 1, None, None) == B.E_SIZE
    # 16-byte alignment of weights, stride and input
    assert L.eidm_matmul_id(ctypes.byref(s), B.DIRECT, P(FAKE + 8), wb, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                            need, None, None) == B.E_ALIGN
    assert L.eidm_matmul_id(ctypes.byref(s), B.DIRECT, P(FAKE), wb, P(FAKE + 4), P(FAKE), P(FAKE), P(FAKE),
                            need, None, None) == B.E_ALIGN
    s2 = B.make_shape(B.BF16, 8, 64, 128, 2, 4, 64 * 128 * 2 + 8, arith=B.ARITH_SPLIT16)
    assert L.eidm_matmul_id(ctypes.byref(s2), B.DIRECT, P(FAKE), wb + 32, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                            need, None, None) == B.E_ALIGN
    assert lib.last_dispatch().dispatch_count == 0
