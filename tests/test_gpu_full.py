"""GPU parity at the benchmark's full sizes, in the launch configuration the
benchmark times (the same ABI calls and routes).  The oracle checks sampled
outputs one by one; Direct and Grouped are compared over the whole output.
"""
import numpy as np
import pytest
import torch

import oracle
from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W

from helpers import assert_close, ids_to_dev, to_dev, u32

pytestmark = pytest.mark.gpu

SAMPLES = 3000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _device_weights(wl):
    w = torch.empty(wl.weight_bytes, dtype=torch.uint8, device="cuda")
    W.fill_weights(wl, w)
    return w


def _packed_experts(wl, experts):
    """Host bytes of the given experts packed densely, in that order."""
    return np.concatenate([W.expert_weights(wl, int(e)).contiguous().view(torch.uint8).numpy().reshape(-1)
                           for e in experts])


def _spot_check(wl, y_gpu, x, ids, samples=SAMPLES, seed=0):
    """Oracle values at random (row, col) pairs, computed on the touched
    experts only (placement independence lets them be packed)."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, wl.routed_rows, samples).astype(np.uint64)
    cols = rng.integers(0, wl.n, samples).astype(np.uint32)
    flat = ids.reshape(-1)
    experts = np.unique(flat[rows.astype(np.int64)])
    remap = {int(e): i for i, e in enumerate(experts)}
    local = np.array([remap.get(int(e), 0) for e in flat], dtype=np.uint32).reshape(ids.shape)
    packed = _packed_experts(wl, experts)
    body = wl.n * wl.k * W.DTYPE_SIZE[wl.dtype]
    ref = oracle.matmul_id_at(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, len(experts), body, wl.layout,
                              packed, x, local, rows, cols)
    got = y_gpu[rows.astype(np.int64), cols.astype(np.int64)]
    return assert_close(got, ref, what=f"{wl.name} sampled y")


def _scratch(lib, wl):
    return torch.empty(lib.query(B.shape_of(wl), B.GROUPED).scratch_bytes, dtype=torch.uint8,
                       device="cuda")


def test_decode_full_path(lib):
    """m=1, top-8 of 256 bf16 experts [1536, 4096]: router ids exact, every
    output vs the oracle, Direct == Grouped over y."""
    wl = W.WORKLOADS["decode"]
    print("[case] decode full path", flush=True)
    wdev = _device_weights(wl)
    x = W.activations(wl)
    logits, bias = W.router_logits(wl), W.router_bias(wl)
    ids = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    gates = torch.empty((1, 8), dtype=torch.float32, device="cuda")
    y = torch.empty((8, wl.n), dtype=torch.float32, device="cuda")
    out = torch.empty((1, wl.n), dtype=torch.float32, device="cuda")
    taken = lib.moe_forward(B.shape_of(wl), B.AUTO, wdev, to_dev(x), to_dev(logits), to_dev(bias), ids,
                            gates, y, out, None, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert taken == B.DIRECT
    ids_o, gates_o, _, _ = oracle.route(logits, bias, 8)
    assert np.array_equal(u32(ids), ids_o)
    # all 8 x 1536 outputs: pack the 8 picked experts
    packed = _packed_experts(wl, ids_o[0])
    y_o = oracle.matmul_id(wl.dtype, 1, wl.n, wl.k, 8, 8, wl.n * wl.k * 2, wl.layout, packed, x,
                           np.arange(8, dtype=np.uint32)[None])
    assert_close(y.cpu().numpy(), y_o, what="decode y")
    assert_close(out.cpu().numpy(), oracle.combine(y_o, gates_o, 8), what="decode out")
    yg = torch.empty_like(y)
    lib.matmul_id(B.shape_of(wl), B.GROUPED, wdev, to_dev(x), ids, yg, _scratch(lib, wl),
                  weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), yg.view(torch.int32))


@pytest.mark.parametrize("name", ["prefill_balanced", "prefill_skewed"])
def test_prefill_profiles_full(lib, name):
    wl = W.WORKLOADS[name]
    print(f"[case] {name} full", flush=True)
    wdev = _device_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    xd, idd = to_dev(x), ids_to_dev(ids)
    yg = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    yd = torch.empty_like(yg)
    lib.matmul_id(B.shape_of(wl), B.GROUPED, wdev, xd, idd, yg, _scratch(lib, wl),
                  weight_bytes=wl.weight_bytes)
    lib.matmul_id(B.shape_of(wl), B.DIRECT, wdev, xd, idd, yd, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int32), yd.view(torch.int32)), "Direct and Grouped differ"
    _spot_check(wl, yg.cpu().numpy(), x, ids)
    # combine with the uniform 1/8 gates, sampled tokens
    out = torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda")
    g = W.gates(wl)
    lib.combine(yg, to_dev(g), out)
    torch.cuda.synchronize()
    toks = np.random.default_rng(3).integers(0, wl.m, 8)
    yh = yg.cpu().numpy().astype(np.float64).reshape(wl.m, wl.top_k, wl.n)
    ref = np.einsum("ts,tsn->tn", g[toks].astype(np.float64), yh[toks])
    assert_close(out.cpu().numpy()[toks], ref, what="combine")


def test_down_projection_full_path(lib):
    """m=2048 tokens, per-slot input [2048, 8, 768], f16 experts [256, 2048, 768],
    sigmoid + bias routing, gate-weighted sum -> [2048, 2048]."""
    wl = W.WORKLOADS["down_proj"]
    print("[case] down projection full path", flush=True)
    wdev = _device_weights(wl)
    x = W.activations(wl)
    logits, bias = W.router_logits(wl), W.router_bias(wl)
    shape = B.shape_of(wl)
    ids = torch.empty((wl.m, 8), dtype=torch.int32, device="cuda")
    gates = torch.empty((wl.m, 8), dtype=torch.float32, device="cuda")
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda")
    taken = lib.moe_forward(shape, B.AUTO, wdev, to_dev(x), to_dev(logits), to_dev(bias), ids, gates,
                            y, out, _scratch(lib, wl), weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert taken == B.GROUPED
    ids_o, gates_o, _, _ = oracle.route(logits, bias, 8)
    assert np.array_equal(u32(ids), ids_o)
    g = gates.cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(g - gates_o) / gates_o)) <= 2e-6
    yh = y.cpu().numpy()
    _spot_check(wl, yh, x, ids_o)
    # out on sampled tokens: the oracle's own y rows for those tokens, combined
    toks = np.random.default_rng(4).integers(0, wl.m, 6)
    experts = np.unique(ids_o[toks])
    remap = {int(e): i for i, e in enumerate(experts)}
    packed = _packed_experts(wl, experts)
    sub_ids = np.array([[remap[int(e)] for e in ids_o[t]] for t in toks], dtype=np.uint32)
    sub_x = x.reshape(wl.m, 8, wl.k)[toks].reshape(-1, wl.k)
    y_o = oracle.matmul_id(wl.dtype, len(toks), wl.n, wl.k, 8, len(experts), wl.n * wl.k * 2,
                           wl.layout, packed, sub_x, sub_ids)
    out_o = oracle.combine(y_o, gates_o[toks], 8)
    assert_close(out.cpu().numpy()[toks], out_o, what="down_proj out")
    # Direct over the same routed ids gives the same bits
    yd = torch.empty_like(y)
    lib.matmul_id(shape, B.DIRECT, wdev, to_dev(x), ids, yd, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), yd.view(torch.int32))
    # every output of y, and every token of out, against the oracle (threaded)
    from helpers import host_threads
    wb = wdev.cpu().numpy()
    y_all = oracle.matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb,
                                     x, ids_o, host_threads())
    err_y = assert_close(yh, y_all, what="down_proj every output of y")
    out_all = oracle.combine(y_all, gates_o, wl.top_k)
    err_o = assert_close(out.cpu().numpy(), out_all, what="down_proj every token of out")
    print(f"[case] down projection: every y max rel err {err_y:.3e}, every out {err_o:.3e}", flush=True)


def test_graph_replays_match_eager(lib):
    """The benchmark replays captured steps: every replay equals the eager result."""
    wl = W.small("down_proj", m=64, n=128, k=256, n_experts=32, top_k=4)
    wdev = to_dev(W.weight_bytes(wl))
    x, logits, bias = to_dev(W.activations(wl)), to_dev(W.router_logits(wl)), to_dev(W.router_bias(wl))
    shape = B.shape_of(wl)
    scratch = _scratch(lib, wl)
    bufs = dict(ids=torch.empty((wl.m, 4), dtype=torch.int32, device="cuda"),
                gates=torch.empty((wl.m, 4), dtype=torch.float32, device="cuda"),
                y=torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda"),
                out=torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda"))

    def step():
        lib.moe_forward(shape, B.GROUPED, wdev, x, logits, bias, bufs["ids"], bufs["gates"], bufs["y"],
                        bufs["out"], scratch, weight_bytes=wl.weight_bytes)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in bufs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for v in bufs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k], eager[k]), f"replay {rep}: {k} differs"
        step()  # eager work between replays
        torch.cuda.synchronize()


def _full_ids_host(wl):
    if wl.ids_kind == "logits":
        ids, _, _, _ = oracle.route(W.router_logits(wl), W.router_bias(wl), wl.top_k)
        return ids
    return W.ids(wl)


@pytest.mark.parametrize("name", ["prefill_balanced", "prefill_skewed", "down_proj"])
def test_full_size_whole_output_equals_the_documented_order(lib, name):
    """Every output of the benchmark's Grouped call equals the CPU evaluation
    of the documented f32 order bit for bit (threaded over the host's cores),
    and for the balanced configuration every output is also within the bar
    of the oracle."""
    from helpers import canonical_matmul_id, host_threads
    wl = W.WORKLOADS[name]
    print(f"[case] whole output {name}", flush=True)
    wdev = _device_weights(wl)
    xh = W.activations(wl)
    ih = _full_ids_host(wl)
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    taken = lib.matmul_id(B.shape_of(wl), B.GROUPED, wdev, to_dev(xh), ids_to_dev(ih), y, _scratch(lib, wl),
                          weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert taken == B.GROUPED
    yg = y.cpu().numpy()
    wb = wdev.cpu().numpy()
    del wdev, y
    threads = host_threads()
    ref = canonical_matmul_id(wl, wb, xh, ih, threads=threads)
    diff = np.flatnonzero(yg.view(np.uint32) != ref.view(np.uint32))
    assert diff.size == 0, f"{diff.size} outputs differ from the documented order, first at {diff[:5]}"
    if name == "prefill_balanced":
        full = oracle.matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb,
                                        xh, ih, threads)
        err = assert_close(yg, full, what=f"{name} every output")
        print(f"[case] {name}: every output vs the oracle, max rel err {err:.3e}", flush=True)
