"""The allocation-free matmul entry point (eidm_matmul_id_noalloc) against
eidm_matmul_id with a caller scratch: bit for bit, on two calls in a row, the
second with a smaller input (the library's static map array keeps the first
call's contents and must not leak them into the second)."""
import numpy as np
import pytest
import torch

from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W

from helpers import ids_to_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _wl(name, dtype, m, n, k, top_k, n_experts, layout=W.LAYOUT_SHARED, seed=7):
    return W.Workload(name, dtype, m, n, k, top_k, n_experts, n * k * W.DTYPE_SIZE[dtype], layout,
                      W.IDS_DISTINCT, seed, 0.05, "random", "softmax")


def _run(lib, wl, route):
    print(f"[case] noalloc {wl.name} route {route}", flush=True)
    shape = B.shape_of(wl)
    w = to_dev(W.weight_bytes(wl))
    x = to_dev(W.activations(wl))
    ids = ids_to_dev(W.ids(wl))
    y_ref = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    y = torch.full((wl.routed_rows, wl.n), float("nan"), dtype=torch.float32, device="cuda")
    scratch = torch.empty(max(1, lib.query(shape, B.GROUPED).scratch_bytes), dtype=torch.uint8, device="cuda")
    taken_ref = lib.matmul_id(shape, route, w, x, ids, y_ref, scratch, weight_bytes=wl.weight_bytes)
    taken = lib.matmul_id_noalloc(shape, route, w, x, ids, y, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert taken == taken_ref
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), f"{wl.name}: outputs differ"
    return taken


@pytest.mark.parametrize("route", [B.GROUPED, B.AUTO, B.DIRECT])
def test_noalloc_matches_the_scratch_entry_point_on_two_calls(lib, route):
    big = _wl("big", W.DT_BF16, 300, 96, 1024, 4, 16, seed=61)     # 16x16x1 Grouped kernel
    small = _wl("small", W.DT_F16, 37, 70, 304, 3, 9, layout=W.LAYOUT_SLOTTED, seed=62)  # earlier kernels
    t1 = _run(lib, big, route)
    t2 = _run(lib, small, route)
    if route == B.GROUPED:
        assert t1 == t2 == B.GROUPED
    if route == B.DIRECT:
        assert t1 == t2 == B.DIRECT


def test_noalloc_down_projection_shape_then_a_smaller_one(lib):
    # the down-projection configuration's shape (16384 routed rows, 256 experts)
    # with random ids, then the first shape again at a tenth of the rows
    full = _wl("down_like", W.DT_F16, 2048, 256, 768, 8, 256, layout=W.LAYOUT_SLOTTED, seed=63)
    _run(lib, full, B.GROUPED)
    _run(lib, full.with_(m=205, name="down_like_small"), B.GROUPED)
