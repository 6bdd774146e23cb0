"""The CPU evaluator of the documented f32 reduction order (the GPU routes
must equal it bit for bit): its threaded form, which regroups rows by expert
for speed at full sizes, gives the same bits as the plain row-by-row form, and
both stay within the parity bar of the exact oracle."""
import numpy as np
import pytest

import oracle
from expert_id_matmul_amd import workloads as W

from helpers import assert_close, canonical_matmul_id


def _wl(name, dtype, m, n, k, top_k, E, layout=W.LAYOUT_SHARED, seed=3):
    return W.Workload(name, dtype, m, n, k, top_k, E, n * k * W.DTYPE_SIZE[dtype] + 64, layout, W.IDS_DISTINCT,
                      seed, 0.05, "random", "softmax")


CASES = [
    _wl("ragged_bf16", W.DT_BF16, 37, 19, 300, 3, 9, seed=31),
    _wl("slotted_f16", W.DT_F16, 21, 33, 136, 4, 6, layout=W.LAYOUT_SLOTTED, seed=32),
    _wl("f32_short_k", W.DT_F32, 40, 10, 8, 2, 5, seed=33),
    _wl("one_expert", W.DT_BF16, 9, 7, 1100, 1, 1, seed=34),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("threads", [2, 5])
def test_threaded_order_equals_row_by_row(wl, threads):
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = W.ids(wl).copy()
    ids[1, 0] = wl.n_experts          # a row naming no expert: NaN in both
    ids[-1, -1] = 0xFFFFFFFF
    plain = canonical_matmul_id(wl, wb, x, ids)
    threaded = canonical_matmul_id(wl, wb, x, ids, threads=threads)
    assert np.array_equal(plain.view(np.uint32), threaded.view(np.uint32))
    bad = {wl.top_k, wl.routed_rows - 1}
    for r in range(wl.routed_rows):
        assert np.isnan(plain[r]).all() == (r in bad)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_documented_order_is_within_the_bar_of_the_oracle(wl):
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    got = canonical_matmul_id(wl, wb, x, ids, threads=3)
    ref = oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb, x, ids)
    assert_close(got, ref, what=wl.name)
