"""Host-side logic of bench.py (no GPU): the cold-expert relabelling, the
algorithmic byte count of a decode step, the one-GPU guard and the
provenance of the HBM traffic figure."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


@pytest.mark.parametrize("seed", range(5))
def test_relabel_is_a_permutation_sending_the_picks_to_the_targets(bench, seed):
    rng = np.random.default_rng(seed)
    n_experts, top_k = 256, 8
    picks = rng.choice(n_experts, size=top_k, replace=False)
    target = np.arange(top_k) + top_k * int(rng.integers(0, n_experts // top_k))
    p = bench._relabel(n_experts, picks, target)
    assert sorted(p.tolist()) == list(range(n_experts))
    assert np.array_equal(p[picks], target)
    # the other experts keep their relative order
    rest = [e for e in range(n_experts) if e not in set(picks.tolist())]
    assert np.all(np.diff(p[rest]) > 0)


def test_relabelled_logits_route_to_the_target_experts(bench):
    """Relabelling the router inputs moves the top-k picks to the target
    labels (checked with the CPU oracle's router on the decode workload)."""
    import oracle
    from expert_id_matmul_amd import workloads as W
    wl = W.WORKLOADS["decode"]
    logits0, bias0 = W.router_logits(wl)[0], W.router_bias(wl)
    ids0, _, _, _ = oracle.route(logits0[None], bias0, wl.top_k)
    picks = ids0[0].astype(np.int64)
    for i in (0, 5, 31):
        target = np.arange(wl.top_k) + wl.top_k * i
        p = bench._relabel(wl.n_experts, picks, target)
        logits = np.empty_like(logits0)
        bias = np.empty_like(bias0)
        logits[p] = logits0
        bias[p] = bias0
        ids, _, _, _ = oracle.route(logits[None], bias, wl.top_k)
        assert np.array_equal(ids[0], target.astype(np.uint32))


def test_decode_algorithmic_bytes(bench):
    from expert_id_matmul_amd import workloads as W
    nb = bench.decode_bytes(W.WORKLOADS["decode"])
    assert nb["touched_weights"] == 8 * 1536 * 4096 * 2 == 100_663_296
    # x 16 KB, logits and bias 1 KB each, y 48 KB, out 6 KB, ids and gates 64 B
    assert nb["algorithmic"] == 100_663_296 + 4096 * 4 + 256 * 4 * 2 + 8 * 1536 * 4 + 1536 * 4 + 8 * 8


def test_percentiles_pick_the_documented_positions(bench):
    v = [5.0, 1.0, 4.0, 2.0, 3.0, 9.0, 7.0, 8.0, 6.0]
    assert bench._percentiles(v) == {"p25": 3.0, "median": 5.0, "p75": 7.0}


def test_more_than_one_gpu_is_refused_with_a_message():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_traffic_summary_names_the_sources_it_was_taken_on(bench):
    """The decode HBM counter summary carries the sha256 of the decode
    kernel's sources; bench.py reports its byte count only while that hash
    equals the hash of the sources built now."""
    fields = {}
    with open(bench.TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    sha = fields["sources_sha256"]
    assert len(sha) == 64 and all(c in "0123456789abcdef" for c in sha)
    assert int(fields["hbm_bytes_per_launch"]) > 0
    if sha == bench.decode_source_hash():
        assert bench.decode_traffic() == int(fields["hbm_bytes_per_launch"])
    else:
        assert bench.decode_traffic() is None
