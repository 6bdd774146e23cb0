"""The split-16 arithmetic on the GPU (16-bit weights exact, activations
split into three 16-bit parts, products on the 16-bit matrix core): Direct
and Grouped bit identical on every shape, both within the 2e-5 bar of the
CPU oracle (mlx-native dense_matmul_id_auto.rs: the value-independence
theorem statement; the f32 result must stay inside the oracle tolerance).

There is no CPU evaluation of the instruction's internal summation, so the
bits themselves are pinned only by Direct == Grouped; the values are pinned
by the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W

from helpers import assert_close, check_guarded, ids_to_dev, poisoned_output, to_dev, u32

pytestmark = pytest.mark.gpu

S16 = B.ARITH_SPLIT16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _wl(name, dtype, m, n, k, top_k, n_experts, stride=None, layout=W.LAYOUT_SHARED, mult=W.IDS_DISTINCT,
        seed=7, ids_kind="random", w_std=0.05):
    return W.Workload(name, dtype, m, n, k, top_k, n_experts, stride or n * k * 2, layout, mult, seed, w_std,
                      ids_kind, "softmax", S16)


SMALL = [
    # k with a step partly past k and a last round of two steps (k = 296)
    _wl("s16_bf16_tail", W.DT_BF16, 37, 70, 296, 3, 9, seed=201),
    _wl("s16_f16_slot_tail", W.DT_F16, 20, 64, 264, 8, 16, layout=W.LAYOUT_SLOTTED, seed=202),
    # many jobs per block, a ragged last column tile (1000 = 7 x 128 + 104)
    _wl("s16_bf16_jobs", W.DT_BF16, 256, 1000, 512, 8, 16, seed=203),
    _wl("s16_f16_jobs_slot", W.DT_F16, 150, 700, 384, 6, 10, layout=W.LAYOUT_SLOTTED, seed=204),
    # one step of 8 k, a job of one round
    _wl("s16_f16_k8", W.DT_F16, 5, 9, 8, 2, 3, seed=205),
    _wl("s16_f16_one_round", W.DT_F16, 64, 200, 128, 4, 4, seed=206),
    _wl("s16_may_repeat", W.DT_BF16, 12, 48, 256, 5, 3, mult=W.IDS_MAY_REPEAT, seed=207, ids_kind="repeat"),
    _wl("s16_decode_like", W.DT_BF16, 1, 136, 1024, 8, 64, seed=208),
    _wl("s16_long_k", W.DT_BF16, 3, 40, 4224, 4, 8, seed=209),
    # padded expert stride (a multiple of 16 bytes)
    _wl("s16_stride_pad", W.DT_BF16, 30, 50, 200, 3, 5, stride=50 * 200 * 2 + 64, seed=210),
    # n below one 16-column tile, one expert
    _wl("s16_one_expert", W.DT_F16, 17, 12, 96, 1, 1, seed=211),
]


def _run(lib, wl, route, w, x, ids):
    shape = B.shape_of(wl)
    scratch = torch.empty(lib.query(shape, route).scratch_bytes, dtype=torch.uint8, device="cuda")
    y = poisoned_output(wl.routed_rows * wl.n)
    taken = lib.matmul_id(shape, route, w, x, ids, y, scratch, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert taken == route
    return y


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_split16_parity_and_bit_identity(lib, wl):
    print(f"[case] split16 {wl.name}", flush=True)
    wb = W.weight_bytes(wl)
    xh = W.activations(wl)
    ih = W.ids(wl)
    w, x, ids = to_dev(wb), to_dev(xh), ids_to_dev(ih)
    yd = _run(lib, wl, B.DIRECT, w, x, ids)
    yg = _run(lib, wl, B.GROUPED, w, x, ids)
    n_out = wl.routed_rows * wl.n
    vd = check_guarded(yd, n_out)
    vg = check_guarded(yg, n_out)
    assert np.array_equal(vd.view(np.uint32), vg.view(np.uint32)), "Direct and Grouped bits differ"
    ref = oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb, xh, ih)
    err = assert_close(vd.reshape(wl.routed_rows, wl.n), ref, what=wl.name)
    print(f"[case] {wl.name} max rel err {err:.3e}", flush=True)


def test_split16_adversarial_activations(lib):
    """The page's calibration activations (bases 1 + 2^-23 and its negative,
    eight values of mixed magnitude): the split is exact for every one of them
    in bf16, and within the bar for f16."""
    for dt in (W.DT_BF16, W.DT_F16):
        wl = _wl(f"s16_adv_{dt}", dt, 64, 96, 1024, 4, 8, seed=212, ids_kind="balanced")
        print(f"[case] split16 adversarial dtype {dt}", flush=True)
        wb = W.weight_bytes(wl)
        xh = W.adversarial_activations(wl.input_rows, wl.k)
        ih = W.ids(wl)
        w, x, ids = to_dev(wb), to_dev(xh), ids_to_dev(ih)
        yd = _run(lib, wl, B.DIRECT, w, x, ids)
        yg = _run(lib, wl, B.GROUPED, w, x, ids)
        n_out = wl.routed_rows * wl.n
        vd, vg = check_guarded(yd, n_out), check_guarded(yg, n_out)
        assert np.array_equal(vd.view(np.uint32), vg.view(np.uint32))
        ref = oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb, xh,
                               ih)
        assert_close(vd.reshape(wl.routed_rows, wl.n), ref, what=wl.name)


def test_split16_ids_naming_no_expert_give_nan_rows(lib):
    wl = _wl("s16_bad_ids", W.DT_BF16, 40, 64, 256, 4, 8, seed=213)
    print("[case] split16 bad ids", flush=True)
    wb = W.weight_bytes(wl)
    xh = W.activations(wl)
    ih = W.ids(wl).copy()
    ih[3, 1] = wl.n_experts
    ih[17, 0] = 0xFFFFFFFF
    w, x, ids = to_dev(wb), to_dev(xh), ids_to_dev(ih)
    outs = []
    for route in (B.DIRECT, B.GROUPED):
        y = _run(lib, wl, route, w, x, ids)
        outs.append(check_guarded(y, wl.routed_rows * wl.n, allow_nan_rows=True).reshape(wl.routed_rows, wl.n))
    vd, vg = outs
    assert np.array_equal(vd.view(np.uint32), vg.view(np.uint32))
    bad = {3 * wl.top_k + 1, 17 * wl.top_k}
    for r in range(wl.routed_rows):
        assert np.isnan(vd[r]).all() == (r in bad)


def test_split16_receipts(lib):
    wl = _wl("s16_receipt", W.DT_BF16, 96, 256, 512, 4, 8, seed=214)
    shape = B.shape_of(wl)
    w, x, ids = to_dev(W.weight_bytes(wl)), to_dev(W.activations(wl)), ids_to_dev(W.ids(wl))
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    for route, kernels in ((B.DIRECT, ["split_x", "direct_split16"]),
                           (B.GROUPED, ["map_split_x", "grouped_split16"])):
        scratch = torch.empty(lib.query(shape, route).scratch_bytes, dtype=torch.uint8, device="cuda")
        lib.matmul_id(shape, route, w, x, ids, y, scratch)
        d = lib.last_dispatch()
        assert d.route == route and d.kernels() == kernels
    torch.cuda.synchronize()


def test_split16_map_too_large_for_one_launch(lib):
    """16,800 routed rows (above the one-launch map's 16,384): the split, the
    two-launch map and the Grouped kernel run separately, with the same bits
    as Direct."""
    wl = _wl("s16_big_map", W.DT_BF16, 4200, 64, 256, 4, 16, seed=215)
    print("[case] split16 two-launch map", flush=True)
    wb = W.weight_bytes(wl)
    xh = W.activations(wl)
    ih = W.ids(wl)
    w, x, ids = to_dev(wb), to_dev(xh), ids_to_dev(ih)
    yd = _run(lib, wl, B.DIRECT, w, x, ids)
    yg = _run(lib, wl, B.GROUPED, w, x, ids)
    assert lib.last_dispatch().kernels() == ["split_x", "map_histogram", "map_scatter", "grouped_split16"]
    n_out = wl.routed_rows * wl.n
    vd, vg = check_guarded(yd, n_out), check_guarded(yg, n_out)
    assert np.array_equal(vd.view(np.uint32), vg.view(np.uint32))
    ref = oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb, xh, ih)
    assert_close(vd.reshape(wl.routed_rows, wl.n), ref, what=wl.name)


# ------------------------------------------------------------- full sizes
def _device_weights(wl):
    t = torch.empty(wl.weight_bytes, dtype=torch.uint8, device="cuda")
    W.fill_weights(wl, t)
    return t


def _spot_check(wl, y, xh, ih, samples=3000, seed=0):
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, wl.routed_rows, samples).astype(np.uint64)
    cols = rng.integers(0, wl.n, samples).astype(np.uint32)
    flat = ih.reshape(-1)
    experts = np.unique(flat[rows.astype(np.int64)])
    remap = {int(e): i for i, e in enumerate(experts)}
    local = np.array([remap.get(int(e), 0) for e in flat], dtype=np.uint32).reshape(ih.shape)
    packed = np.concatenate([W.expert_weights(wl, int(e)).contiguous().view(torch.uint8).numpy().reshape(-1)
                             for e in experts])
    body = wl.n * wl.k * 2
    ref = oracle.matmul_id_at(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, len(experts), body, wl.layout, packed, xh,
                              local, rows, cols)
    got = y[rows.astype(np.int64), cols.astype(np.int64)]
    return assert_close(got, ref, what=f"{wl.name} sampled y")


def _full_ids(wl):
    if wl.ids_kind == "logits":
        ids, _, _, _ = oracle.route(W.router_logits(wl), W.router_bias(wl), wl.top_k)
        return ids
    return W.ids(wl)


@pytest.mark.parametrize("name", ["prefill_balanced", "prefill_skewed", "down_proj", "decode"])
def test_split16_full_size(lib, name):
    """The benchmark configurations in the split-16 arithmetic: Direct ==
    Grouped over the whole output; every output of the three prefill
    configurations against the oracle (decode: sampled outputs)."""
    wl = W.WORKLOADS[name].with_(arith=S16)
    print(f"[case] split16 full {name}", flush=True)
    w = _device_weights(wl)
    xh = W.activations(wl)
    ih = _full_ids(wl)
    x, ids = to_dev(xh), ids_to_dev(ih)
    shape = B.shape_of(wl)
    ys = []
    for route in (B.GROUPED, B.DIRECT):
        scratch = torch.empty(lib.query(shape, route).scratch_bytes, dtype=torch.uint8, device="cuda")
        y = torch.full((wl.routed_rows, wl.n), float("nan"), dtype=torch.float32, device="cuda")
        lib.matmul_id(shape, route, w, x, ids, y, scratch, weight_bytes=wl.weight_bytes)
        torch.cuda.synchronize()
        ys.append(y)
        del scratch
    assert torch.equal(ys[0].view(torch.int32), ys[1].view(torch.int32)), "Direct and Grouped bits differ"
    yh = ys[0].cpu().numpy()
    assert np.isfinite(yh).all()
    if name == "decode":
        err = _spot_check(wl, yh, xh, ih)
        print(f"[case] split16 full {name} sampled max rel err {err:.3e}", flush=True)
    else:
        # every output against the oracle, threaded over the host's cores
        from helpers import host_threads
        wb = w.cpu().numpy()
        ref = oracle.matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout,
                                       wb, xh, ih, host_threads())
        err = assert_close(yh, ref, what=f"{name} split16 every output")
        print(f"[case] split16 full {name} every output max rel err {err:.3e}", flush=True)
    del w, ys
    torch.cuda.empty_cache()


@pytest.mark.parametrize("route", [B.GROUPED, B.DIRECT])
def test_split16_graph_replays_match_eager(lib, route):
    """A captured split-16 call (Grouped: the map-and-split launch and the
    Grouped kernel; Direct: split and Direct) replays to the eager bits, with
    eager calls and synchronisations between the replays."""
    wl = _wl("s16_graph", W.DT_BF16, 96, 256, 512, 4, 8, seed=216)
    print(f"[case] split16 graph route {route}", flush=True)
    shape = B.shape_of(wl)
    w, x, ids = to_dev(W.weight_bytes(wl)), to_dev(W.activations(wl)), ids_to_dev(W.ids(wl))
    scratch = torch.empty(lib.query(shape, route).scratch_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")

    def step():
        lib.matmul_id(shape, route, w, x, ids, y, scratch, weight_bytes=wl.weight_bytes)

    step()
    torch.cuda.synchronize()
    eager = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        y.zero_()
        scratch.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), eager.view(torch.int32)), f"replay {rep} differs"
        step()
        torch.cuda.synchronize()
