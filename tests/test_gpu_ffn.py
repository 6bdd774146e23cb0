"""The expert FFN (route -> gate/up matmul_id -> silu * up -> down matmul_id
-> combine) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W
from helpers import assert_close, to_dev, u32

pytestmark = pytest.mark.gpu

SMALL = [W.FfnWorkload("ffn_bf16", W.DT_BF16, 37, 96, 72, 4, 12, 51, 0.05),
         W.FfnWorkload("ffn_f16_ragged", W.DT_F16, 23, 130, 61, 3, 9, 52, 0.05),
         W.FfnWorkload("ffn_f32", W.DT_F32, 16, 64, 48, 2, 6, 53, 0.1),
         W.FfnWorkload("ffn_many_rows", W.DT_BF16, 200, 256, 256, 8, 16, 54, 0.03),
         # gate/up k = 2880 (23 rounds, the last partly past k), down k = 1408 (11 rounds)
         W.FfnWorkload("ffn_odd_rounds_tail", W.DT_BF16, 64, 2880, 1408, 4, 8, 55, 0.02)]


def _device_weights(fw):
    out = {}
    for w in ("gate", "up", "down"):
        p = fw.part(w)
        t = torch.empty(p.weight_bytes, dtype=torch.uint8, device="cuda")
        W.fill_weights(p, t)
        out[w] = t
    return out


def _run(lib, fw, wdev, x, logits, bias, route):
    shape = B.ffn_shape_of(fw)
    ids = torch.empty((fw.m, fw.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((fw.m, fw.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((fw.m, fw.hidden), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.moe_ffn_scratch_bytes(shape), dtype=torch.uint8, device="cuda")
    taken = lib.moe_ffn(shape, route, wdev["gate"], wdev["up"], wdev["down"], x, logits, bias, ids, gates,
                        out, scratch)
    torch.cuda.synchronize()
    return taken, ids, gates, out


@pytest.mark.parametrize("fw", SMALL, ids=lambda f: f.name)
def test_ffn_matches_the_oracle_and_both_routes_agree_bitwise(lib, fw):
    print(f"[case] ffn {fw.name}", flush=True)
    wdev = _device_weights(fw)
    xh, lh, bh = W.ffn_inputs(fw)
    x, logits, bias = to_dev(xh), to_dev(lh), to_dev(bh)
    t_d, ids_d, gates_d, out_d = _run(lib, fw, wdev, x, logits, bias, B.DIRECT)
    t_g, ids_g, gates_g, out_g = _run(lib, fw, wdev, x, logits, bias, B.GROUPED)
    assert (t_d, t_g) == (B.DIRECT, B.GROUPED)
    assert torch.equal(out_d.view(torch.int32), out_g.view(torch.int32))
    ids_o, gates_o, _, _ = oracle.route(lh, bh, fw.top_k)
    assert np.array_equal(u32(ids_d), ids_o)
    parts = {w: fw.part(w) for w in ("gate", "up", "down")}
    raw = {w: t.cpu().numpy() for w, t in wdev.items()}
    want, _ = oracle.moe_ffn(fw.dtype, fw.m, fw.hidden, fw.inter, fw.top_k, fw.n_experts,
                             parts["gate"].stride, parts["down"].stride, raw["gate"], raw["up"], raw["down"],
                             xh, ids_o, gates_o)
    assert_close(out_d.cpu().numpy(), want, what=f"{fw.name} out")


def test_ffn_prefill_full_size_sampled_tokens(lib):
    """The prefill FFN (m=512, hidden 2048, inter 768, top-8 of 128 bf16
    experts) against the oracle on sampled tokens (tokens are independent)."""
    fw = W.FFN_WORKLOADS["ffn_prefill"]
    print("[case] ffn prefill full size", flush=True)
    wdev = _device_weights(fw)
    xh, lh, bh = W.ffn_inputs(fw)
    taken, ids, gates, out = _run(lib, fw, wdev, to_dev(xh), to_dev(lh), to_dev(bh), B.AUTO)
    assert taken == B.GROUPED
    ids_o, gates_o, _, _ = oracle.route(lh, bh, fw.top_k)
    assert np.array_equal(u32(ids), ids_o)
    tokens = np.array([0, 1, 77, 255, 300, 511])
    parts = {w: fw.part(w) for w in ("gate", "up", "down")}
    raw = {w: t.cpu().numpy() for w, t in wdev.items()}
    want, _ = oracle.moe_ffn(fw.dtype, len(tokens), fw.hidden, fw.inter, fw.top_k, fw.n_experts,
                             parts["gate"].stride, parts["down"].stride, raw["gate"], raw["up"], raw["down"],
                             xh[tokens], ids_o[tokens], gates_o[tokens])
    assert_close(out.cpu().numpy()[tokens], want, what="ffn prefill sampled tokens")


def test_ffn_prefill_full_size_every_token(lib):
    """The same FFN over every token against the oracle (tokens are
    independent, so the oracle runs on chunks of tokens on the host's cores),
    and the Direct route's output equal to the Grouped route's bit for bit."""
    from concurrent.futures import ThreadPoolExecutor
    from helpers import host_threads
    fw = W.FFN_WORKLOADS["ffn_prefill"]
    print("[case] ffn prefill full size, every token", flush=True)
    wdev = _device_weights(fw)
    xh, lh, bh = W.ffn_inputs(fw)
    x, logits, bias = to_dev(xh), to_dev(lh), to_dev(bh)
    taken, ids, gates, out = _run(lib, fw, wdev, x, logits, bias, B.GROUPED)
    assert taken == B.GROUPED
    taken_d, ids_d, _, out_d = _run(lib, fw, wdev, x, logits, bias, B.DIRECT)
    assert taken_d == B.DIRECT and torch.equal(ids, ids_d)
    assert torch.equal(out.view(torch.int32), out_d.view(torch.int32)), "Direct and Grouped FFN outputs differ"
    ids_o, gates_o, _, _ = oracle.route(lh, bh, fw.top_k)
    assert np.array_equal(u32(ids), ids_o)
    parts = {w: fw.part(w) for w in ("gate", "up", "down")}
    raw = {w: t.cpu().numpy() for w, t in wdev.items()}
    chunks = np.array_split(np.arange(fw.m), host_threads())

    def run(tok):
        want, _ = oracle.moe_ffn(fw.dtype, len(tok), fw.hidden, fw.inter, fw.top_k, fw.n_experts,
                                 parts["gate"].stride, parts["down"].stride, raw["gate"], raw["up"], raw["down"],
                                 xh[tok], ids_o[tok], gates_o[tok])
        return want

    with ThreadPoolExecutor(len(chunks)) as ex:
        want = np.concatenate(list(ex.map(run, chunks)))
    err = assert_close(out.cpu().numpy(), want, what="ffn prefill every token")
    print(f"[case] ffn prefill every token: max rel err {err:.3e}", flush=True)


@pytest.mark.parametrize("fw", [SMALL[3], SMALL[4]], ids=lambda f: f.name)
def test_ffn_graph_replays_match_eager(lib, fw):
    """A captured expert-FFN step (route, one shared map, three Grouped
    projections, SiLU·up, combine) replays to the eager bits, with eager
    steps and synchronisations between the replays (the 4x4x1 streamed
    kernel at k = 256, the 16x16x1 kernel at k = 2880 and 1408)."""
    print(f"[case] ffn graph {fw.name}", flush=True)
    wdev = _device_weights(fw)
    xh, lh, bh = W.ffn_inputs(fw)
    x, logits, bias = to_dev(xh), to_dev(lh), to_dev(bh)
    shape = B.ffn_shape_of(fw)
    ids = torch.empty((fw.m, fw.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((fw.m, fw.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((fw.m, fw.hidden), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.moe_ffn_scratch_bytes(shape), dtype=torch.uint8, device="cuda")

    def step():
        lib.moe_ffn(shape, B.GROUPED, wdev["gate"], wdev["up"], wdev["down"], x, logits, bias, ids, gates, out,
                    scratch)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
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
        out.zero_()
        scratch.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {rep} differs"
        step()
        torch.cuda.synchronize()
