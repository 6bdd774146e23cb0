"""Activation-time route calibration and the frozen plan on the GPU
(mlx-native dense_matmul_id_auto.rs: fn calibrate_one_inner and its winner
rule, fn resolve_dense_matmul_id_auto_route)."""
import numpy as np
import pytest
import torch

from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W
from helpers import to_dev, ids_to_dev

pytestmark = pytest.mark.gpu


def rule(rec):
    """The page's winner rule, recomputed from the receipt's own numbers."""
    if not rec.grouped_legal:
        return B.DIRECT
    for p in range(2):
        if not (rec.grouped_wall_median[p] <= 0.95 * rec.direct_wall_median[p]):
            return B.DIRECT
        if not (rec.grouped_wall_p75[p] < rec.direct_wall_p25[p]):
            return B.DIRECT
        if not (rec.grouped_gpu_median[p] <= 1.02 * rec.direct_gpu_median[p]):
            return B.DIRECT
    return B.GROUPED


def _setup(lib, dtype, m, n, k, top_k, E, seed):
    wl = W.Workload("cal", dtype, m, n, k, top_k, E, n * k * W.DTYPE_SIZE[dtype], W.LAYOUT_SHARED,
                    W.IDS_DISTINCT, seed, 0.02, "random", "uniform")
    weights = torch.empty(wl.weight_bytes, dtype=torch.uint8, device="cuda")
    W.fill_weights(wl, weights)
    plan = B.Plan(lib)
    shape = B.shape_of(wl)
    ws = torch.empty(plan.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    return wl, weights, plan, shape, ws


@pytest.mark.parametrize("name,m,n,k,top_k,E", [
    ("decode_like", 1, 512, 1024, 8, 64),
    ("prefill_like", 256, 512, 1024, 8, 32),
])
def test_calibration_follows_the_rule_and_serves_the_plan(lib, name, m, n, k, top_k, E):
    print(f"[case] calibrate {name}", flush=True)
    wl, weights, plan, shape, ws = _setup(lib, W.DT_BF16, m, n, k, top_k, E, seed=80)
    rec = plan.calibrate(shape, weights, ws, weight_bytes=wl.weight_bytes)
    print("[case] receipt", {k_: v for k_, v in rec.as_dict().items() if k_ != "reserved0"}, flush=True)
    assert rec.grouped_legal == 1
    assert rec.bit_identical == 1, B.CAL_REASONS[rec.reason]
    assert rec.reason not in (2, 3)
    assert rec.route == rule(rec)
    assert (rec.reason == 0) == (rec.route == B.GROUPED)
    for p in range(2):
        assert 0 < rec.direct_gpu_median[p] <= rec.direct_wall_p75[p] + 1e3
        assert rec.direct_wall_p25[p] <= rec.direct_wall_median[p] <= rec.direct_wall_p75[p]
        assert rec.grouped_wall_p25[p] <= rec.grouped_wall_median[p] <= rec.grouped_wall_p75[p]
    if name == "decode_like":
        assert rec.route == B.DIRECT  # one token: Grouped adds the map and serialises the experts

    # lookups: exact shape -> stored route; same base, unseen m -> Direct; other n -> error
    assert plan.route(shape) == rec.route
    other_m = B.shape_of(wl.with_(m=m + 3))
    assert plan.route(other_m) == B.DIRECT
    with pytest.raises(B.EidmError) as e:
        plan.route(B.shape_of(wl.with_(n=n + 8, stride=(n + 8) * k * 2)))
    assert e.value.code == B.E_UNSUPPORTED

    # the planned call runs the stored route and gives the same bits as both routes
    x = to_dev(W.activations(wl))
    ids = ids_to_dev(W.random_distinct_ids(wl))
    y = torch.empty((wl.routed_rows, n), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.query(shape, B.GROUPED).scratch_bytes, dtype=torch.uint8, device="cuda")
    taken = plan.matmul_id(shape, weights, x, ids, y, scratch, weight_bytes=wl.weight_bytes)
    assert taken == rec.route
    for route in (B.DIRECT, B.GROUPED):
        y2 = torch.empty_like(y)
        lib.matmul_id(shape, route, weights, x, ids, y2, scratch, weight_bytes=wl.weight_bytes)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))

    plan.freeze()
    with pytest.raises(B.EidmError) as e:
        plan.calibrate(shape, weights, ws, weight_bytes=wl.weight_bytes)
    assert e.value.code == B.E_INVALID
    assert plan.route(shape) == rec.route


def _section(ws, offset, count, dtype):
    return ws[offset: offset + count * 4].cpu().numpy().view(dtype)


def _layout(wl):
    """Workspace sections of eidm_calibrate: activations, then the two id
    tables, each at a 256-byte boundary."""
    a = lambda v: (v + 255) // 256 * 256
    x = 0
    ids0 = a(x + wl.input_rows * wl.k * 4)
    ids1 = a(ids0 + wl.routed_rows * 4)
    return x, ids0, ids1


@pytest.mark.parametrize("mult", [W.IDS_DISTINCT, W.IDS_MAY_REPEAT])
def test_calibration_inputs_follow_the_page(lib, mult):
    """fn calibration_buffers: the adversarial activations; distinct ids
    calibrate on balanced (t+s) mod E and skewed s, ids that may repeat on
    t mod E for both profiles.  One complete gate is 27 host waits."""
    top_k, E = (6, 4) if mult == W.IDS_MAY_REPEAT else (4, 16)
    print(f"[case] calibrate inputs mult={mult}", flush=True)
    wl = W.Workload("cal_in", W.DT_BF16, 96, 128, 512, top_k, E, 128 * 512 * 2, W.LAYOUT_SHARED, mult, 81, 0.02,
                    "random", "uniform")
    weights = torch.empty(wl.weight_bytes, dtype=torch.uint8, device="cuda")
    W.fill_weights(wl, weights)
    plan = B.Plan(lib)
    shape = B.shape_of(wl)
    ws = torch.empty(plan.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    rec = plan.calibrate(shape, weights, ws, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    print("[case] receipt", rec.as_dict(), flush=True)
    assert rec.grouped_legal == 1 and rec.bit_identical == 1
    assert rec.reason not in (2, 3, B.CAL_BUDGET)
    assert rec.submissions == B.GATE_SUBMISSIONS
    assert rec.route == rule(rec)
    x0, i0, i1 = _layout(wl)
    x = _section(ws, x0, wl.input_rows * wl.k, np.float32).reshape(wl.input_rows, wl.k)
    assert np.array_equal(x.view(np.uint32), W.adversarial_activations(wl.input_rows, wl.k).view(np.uint32))
    t = np.arange(wl.m)[:, None]
    s = np.arange(top_k)[None, :]
    ids0 = _section(ws, i0, wl.routed_rows, np.uint32).reshape(wl.m, top_k)
    ids1 = _section(ws, i1, wl.routed_rows, np.uint32).reshape(wl.m, top_k)
    if mult == W.IDS_MAY_REPEAT:
        want0 = want1 = np.broadcast_to(t % E, (wl.m, top_k))
    else:
        want0 = (t + s) % E
        want1 = np.broadcast_to(s, (wl.m, top_k))
    assert np.array_equal(ids0, want0) and np.array_equal(ids1, want1)


def test_submission_budget_and_deadline_downgrade(lib):
    """Budget rules on the GPU: a plan with room for exactly one gate
    calibrates one shape and gives the next Direct without GPU work; a plan
    frozen after its deadline turns its Grouped entries into Direct
    (fn downgrade_grouped_after_deadline)."""
    import time
    # many routed rows over few experts: Grouped reads each expert's weights once
    wl, weights, plan, shape, ws = _setup(lib, W.DT_BF16, 2048, 512, 1024, 8, 64, seed=82)
    print("[case] calibrate budget", flush=True)
    plan.set_limits(max_elapsed_ms=60000, max_cases=4, max_submissions=B.GATE_SUBMISSIONS)
    rec = plan.calibrate(shape, weights, ws, weight_bytes=wl.weight_bytes)
    print("[case] receipt", rec.as_dict(), flush=True)
    assert rec.submissions == B.GATE_SUBMISSIONS and rec.bit_identical == 1
    assert rec.route == B.GROUPED, B.CAL_REASONS[rec.reason]
    other = B.shape_of(wl.with_(m=1024))
    rec2 = plan.calibrate(other, weights, ws, weight_bytes=wl.weight_bytes)
    assert (rec2.route, rec2.reason, rec2.submissions) == (B.DIRECT, B.CAL_BUDGET, 0)
    assert plan.freeze() == 0  # before the deadline: nothing changes
    assert plan.route(shape) == B.GROUPED

    plan2 = B.Plan(lib)
    deadline_ms = 3000
    plan2.set_limits(max_elapsed_ms=deadline_ms)
    t0 = time.monotonic()
    rec = plan2.calibrate(shape, weights, ws, weight_bytes=wl.weight_bytes)
    assert rec.route == B.GROUPED, B.CAL_REASONS[rec.reason]
    assert plan2.route(shape) == B.GROUPED
    time.sleep(max(0.0, deadline_ms / 1000 + 0.1 - (time.monotonic() - t0)))
    assert plan2.freeze() == 1
    assert plan2.route(shape) == B.DIRECT
    torch.cuda.synchronize()
