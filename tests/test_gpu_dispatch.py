"""Dispatch receipts on the GPU: which kernels each entry point enqueued, in
order, and the launch geometry it chose (mlx-native dense_matmul_id_auto.rs:
the primitive's receipt {route, dispatch count}, fn expected_dispatches and
the geometry check after each encode).  Direct is one launch; Grouped is the
id -> row map (one launch, or two for large maps) and the Grouped kernel;
the later projections of the expert FFN reuse the first one's map."""
import ctypes
import threading

import pytest
import torch

from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W
from helpers import ids_to_dev, to_dev

pytestmark = pytest.mark.gpu

MAP_KERNELS = (["map_one_pass"], ["map_histogram", "map_scatter"])


def _wl(name, dtype, m, n, k, top_k, E, seed=5, layout=W.LAYOUT_SHARED):
    return W.Workload(name, dtype, m, n, k, top_k, E, n * k * W.DTYPE_SIZE[dtype], layout, W.IDS_DISTINCT, seed,
                      0.05, "random", "softmax")


def _buffers(wl):
    w = to_dev(W.weight_bytes(wl))
    x = to_dev(W.activations(wl))
    ids = ids_to_dev(W.ids(wl))
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    return w, x, ids, y


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _check_map(launches, wl):
    """The map's launches: one block per expert plus the invalid bucket, or
    the two-launch form with equal grids."""
    if len(launches) == 1:
        assert launches[0].grid == wl.n_experts + 1
    else:
        assert launches[0].grid == launches[1].grid >= 1
        assert launches[0].block == launches[1].block and launches[0].block % 64 == 0


def _check_direct(launch, wl):
    """Direct: one block per routed row and group of block/64 * 8 columns; the
    activation row is staged in LDS (4 bytes per element) or not at all."""
    cols = launch.block // 64 * 8
    assert launch.grid == -(-wl.n // cols) * wl.routed_rows
    assert launch.lds_bytes in (0, wl.k * 4)


def _check_grouped16(launch, wl):
    """16x16x1 Grouped: 256 threads, a grid of at most one block per compute
    unit (rounded up to the 8 XCDs) and no more than its job bound, three
    32-row activation buffers in LDS."""
    job_bound = (wl.routed_rows // 32 + wl.n_experts + 1) * -(-wl.n // 64)
    want = min(job_bound, _cus())
    assert launch.block == 256
    assert launch.grid == -(-want // 8) * 8
    assert 3 * 32 * 528 <= launch.lds_bytes <= 160 * 1024


def _receipt(lib, route, n_kernels=None):
    d = lib.last_dispatch()
    assert d.route == route
    assert d.recorded == min(d.dispatch_count, B.MAX_RECORDED_LAUNCHES)
    if n_kernels is not None:
        assert d.dispatch_count == n_kernels
    return d, d.kernels(), [d.launches[i] for i in range(d.recorded)]


@pytest.mark.parametrize("dtype", [W.DT_BF16, W.DT_F16])
def test_matmul_id_receipts_and_geometry(lib, dtype):
    wl = _wl("receipt16", dtype, 300, 96, 1024, 4, 16)
    print(f"[case] receipt matmul_id dtype {dtype}", flush=True)
    shape = B.shape_of(wl)
    w, x, ids, y = _buffers(wl)
    scratch = torch.empty(lib.query(shape, B.GROUPED).scratch_bytes, dtype=torch.uint8, device="cuda")

    assert lib.matmul_id(shape, B.DIRECT, w, x, ids, y, scratch) == B.DIRECT
    _, kernels, launches = _receipt(lib, B.DIRECT, 1)
    assert kernels == ["direct"]
    _check_direct(launches[0], wl)

    assert lib.matmul_id(shape, B.GROUPED, w, x, ids, y, scratch) == B.GROUPED
    d, kernels, launches = _receipt(lib, B.GROUPED)
    assert kernels[-1] == "grouped_16x16" and kernels[:-1] in MAP_KERNELS
    _check_map(launches[:-1], wl)
    _check_grouped16(launches[-1], wl)

    # the allocation-free entry point runs the same launches
    assert lib.matmul_id_noalloc(shape, B.GROUPED, w, x, ids, y) == B.GROUPED
    d2, kernels2, launches2 = _receipt(lib, B.GROUPED, d.dispatch_count)
    assert kernels2 == kernels
    assert [(l.grid, l.block, l.lds_bytes) for l in launches2] == [(l.grid, l.block, l.lds_bytes) for l in launches]
    torch.cuda.synchronize()


def test_f32_and_short_k_use_the_4x4_grouped_kernels(lib):
    cases = [(_wl("f32", W.DT_F32, 200, 64, 512, 4, 8), "grouped_stream"),
             (_wl("short_k", W.DT_BF16, 200, 64, 40, 4, 8), "grouped_job")]  # one round of k
    for wl, kernel in cases:
        print(f"[case] receipt {wl.name}", flush=True)
        shape = B.shape_of(wl)
        w, x, ids, y = _buffers(wl)
        scratch = torch.empty(lib.query(shape, B.GROUPED).scratch_bytes, dtype=torch.uint8, device="cuda")
        lib.matmul_id(shape, B.GROUPED, w, x, ids, y, scratch)
        _, kernels, launches = _receipt(lib, B.GROUPED)
        assert kernels[-1] == kernel and kernels[:-1] in MAP_KERNELS
        assert launches[-1].grid % 8 == 0 and launches[-1].block % 64 == 0
    torch.cuda.synchronize()


def test_moe_forward_receipts(lib):
    wl = _wl("moe", W.DT_BF16, 96, 128, 512, 4, 16)
    print("[case] receipt moe_forward", flush=True)
    shape = B.shape_of(wl)
    w, x, _, y = _buffers(wl)
    logits = to_dev(W.router_logits(wl))
    ids = torch.empty((wl.m, wl.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((wl.m, wl.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.query(shape, B.GROUPED).scratch_bytes, dtype=torch.uint8, device="cuda")

    # Direct with top_k <= 16: route, matmul and combine in one launch
    assert lib.moe_forward(shape, B.DIRECT, w, x, logits, None, ids, gates, y, out, scratch) == B.DIRECT
    _, kernels, launches = _receipt(lib, B.DIRECT, 1)
    assert kernels == ["fused_decode"]
    assert launches[0].block == 64 * wl.top_k

    assert lib.moe_forward(shape, B.GROUPED, w, x, logits, None, ids, gates, y, out, scratch) == B.GROUPED
    _, kernels, launches = _receipt(lib, B.GROUPED)
    assert kernels[0] == "route" and kernels[-2:] == ["grouped_16x16", "combine"]
    assert kernels[1:-2] in MAP_KERNELS
    assert launches[0].grid == -(-wl.m // 4)  # four tokens per router block
    _check_grouped16(launches[-2], wl)
    torch.cuda.synchronize()


def test_moe_ffn_builds_the_map_once(lib):
    # hidden 512 and inter 384: every projection has three or more 128-wide k rounds
    fw = W.FfnWorkload("ffn_receipt", W.DT_BF16, 64, 512, 384, 4, 8, 58, 0.03)
    print("[case] receipt moe_ffn", flush=True)
    shape = B.ffn_shape_of(fw)
    wdev = {}
    for name in ("gate", "up", "down"):
        p = fw.part(name)
        wdev[name] = torch.empty(p.weight_bytes, dtype=torch.uint8, device="cuda")
        W.fill_weights(p, wdev[name])
    xh, lh, bh = W.ffn_inputs(fw)
    x, logits, bias = to_dev(xh), to_dev(lh), to_dev(bh)
    ids = torch.empty((fw.m, fw.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((fw.m, fw.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((fw.m, fw.hidden), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.moe_ffn_scratch_bytes(shape), dtype=torch.uint8, device="cuda")

    lib.moe_ffn(shape, B.DIRECT, wdev["gate"], wdev["up"], wdev["down"], x, logits, bias, ids, gates, out, scratch)
    _, kernels, _ = _receipt(lib, B.DIRECT, 6)
    assert kernels == ["route", "direct", "direct", "silu_mul", "direct", "combine"]

    lib.moe_ffn(shape, B.GROUPED, wdev["gate"], wdev["up"], wdev["down"], x, logits, bias, ids, gates, out,
                scratch)
    _, kernels, _ = _receipt(lib, B.GROUPED)
    assert kernels[0] == "route"
    tail = kernels[-5:]
    assert tail == ["grouped_16x16", "grouped_16x16", "silu_mul", "grouped_16x16", "combine"]
    assert kernels[1:-5] in MAP_KERNELS  # one map for the three projections
    torch.cuda.synchronize()


def test_receipts_are_per_thread_and_reset_by_each_call(lib):
    wl = _wl("thread", W.DT_BF16, 64, 64, 256, 2, 8)
    shape = B.shape_of(wl)
    w, x, ids, y = _buffers(wl)
    lib.matmul_id(shape, B.DIRECT, w, x, ids, y)
    other = {}

    def run():
        lib.matmul_id(shape, B.DIRECT, w, x, ids, y)
        lib.combine(y.view(wl.m, wl.top_k, wl.n), torch.ones((wl.m, wl.top_k), device="cuda"),
                    torch.empty((wl.m, wl.n), device="cuda"))
        other["kernels"] = lib.last_dispatch().kernels()

    t = threading.Thread(target=run)
    t.start()
    t.join()
    assert other["kernels"] == ["combine"]
    assert lib.last_dispatch().kernels() == ["direct"]
    # a call rejected on the host (an unknown route) starts an empty receipt
    P = ctypes.c_void_p
    assert lib.lib.eidm_matmul_id(ctypes.byref(shape), 7, P(w.data_ptr()), wl.weight_bytes, P(x.data_ptr()),
                                  P(ids.data_ptr()), P(y.data_ptr()), None, 0, None, None) == B.E_INVALID
    d = lib.last_dispatch()
    assert (d.route, d.dispatch_count, d.recorded) == (0, 0, 0)
    torch.cuda.synchronize()
