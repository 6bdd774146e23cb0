"""Expert matrices larger than 4 GiB, and experts that start past the first 4 GiB of the weight
buffer: the Grouped kernel's 64-bit weight addressing (its 32-bit lane offsets only cover an
expert under 4 GiB) and the Direct kernel's 64-bit expert offsets.

Two experts of n x k just over 4 GiB each, every token routed to both. Every output is checked
Direct against Grouped bit for bit; sampled outputs, biased to the last columns (the largest
offsets), are checked against the oracle and against the canonical-order emulator. Each sample
is its own one-column problem (that weight row, the token's activation row), so no 8 GiB host
copy is needed. The weights are drawn on the device; the checks read back the bits the kernels
read.
"""
import numpy as np
import pytest
import torch

import oracle
from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W

from helpers import TOL, canonical_matmul_id, check_guarded, ids_to_dev, poisoned_output, to_dev

pytestmark = pytest.mark.gpu

EXTRA_COLUMNS = 40  # n * k * size exceeds 4 GiB by 40 rows


def _small_wl(dtype, k):
    size = W.DTYPE_SIZE[dtype]
    return W.Workload("one_column", dtype, 1, 1, k, 1, 1, k * size, W.LAYOUT_SHARED, W.IDS_DISTINCT,
                      0, 0.0, "random", "softmax")


# The Grouped kernel streams the rounds: 64 of them, 63 (an odd number: jobs
# start on alternate rounds), and 63 with the last one partly past k
@pytest.mark.parametrize("dtype,K", [(W.DT_BF16, 8192), (W.DT_F32, 8192), (W.DT_BF16, 8064), (W.DT_BF16, 7944)],
                         ids=["bf16", "f32", "bf16_odd_rounds", "bf16_odd_rounds_tail"])
def test_experts_larger_than_4_gib(lib, dtype, K):
    torch.cuda.set_device(0)
    size = W.DTYPE_SIZE[dtype]
    n = (1 << 32) // (K * size) + EXTRA_COLUMNS
    n_experts, top_k, m = 2, 2, 8
    stride = n * K * size
    total = n_experts * stride
    assert n * K * size > (1 << 32) and stride > (1 << 32)
    if torch.cuda.mem_get_info()[0] < total + (2 << 30):
        pytest.skip("not enough free device memory for two experts of more than 4 GiB")
    print(f"[case] large experts: dtype={W.DTYPE_NAME[dtype]} n={n} k={K} stride={stride}", flush=True)

    torch.manual_seed(90 + dtype)
    weights = torch.empty(total, dtype=torch.uint8, device="cuda")
    typed = weights.view(torch.float32 if dtype == W.DT_F32 else torch.bfloat16)
    typed.normal_(0.0, 0.02)
    x = W.random_f32((m, K), 91 + dtype)
    ids = np.tile(np.array([0, 1], dtype=np.uint32), (m, 1))   # every token to both experts
    shape = B.make_shape(dtype, m, n, K, top_k, n_experts, stride)

    def run(route):
        out = poisoned_output(m * top_k * n)
        scratch = None
        if route == B.GROUPED:
            scratch = torch.empty(lib.query(shape, B.GROUPED).scratch_bytes, dtype=torch.uint8,
                                  device="cuda")
        taken = lib.matmul_id(shape, route, weights, to_dev(x), ids_to_dev(ids), out, scratch,
                              weight_bytes=total)
        assert taken == route
        torch.cuda.synchronize()
        return check_guarded(out, m * top_k * n).reshape(m * top_k, n)

    yd = run(B.DIRECT)
    yg = run(B.GROUPED)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32)), "Direct and Grouped differ"

    rng = np.random.default_rng(92 + dtype)
    rows = rng.integers(0, m * top_k, size=48)
    cols = np.concatenate([rng.integers(0, n, size=24), n - 1 - rng.integers(0, 64, size=24)])
    swl = _small_wl(dtype, K)
    for r, j in zip(rows.tolist(), cols.tolist()):
        t, s = divmod(r, top_k)
        e = int(ids[t, s])
        begin = e * stride + j * K * size
        row_bytes = weights[begin:begin + K * size].cpu().numpy()
        xr = x[t:t + 1]
        one = np.zeros((1, 1), dtype=np.uint32)
        ref = oracle.matmul_id(dtype, 1, 1, K, 1, 1, K * size, W.LAYOUT_SHARED, row_bytes, xr, one)[0, 0]
        got = float(yd[r, j])
        assert abs(got - ref) / max(1.0, abs(ref)) <= TOL, f"y[{r},{j}] = {got} against the oracle {ref}"
        canon = canonical_matmul_id(swl, row_bytes, xr, one)[0, 0]
        assert np.float32(got).view(np.uint32) == np.float32(canon).view(np.uint32), \
            f"y[{r},{j}] differs from the canonical order"
    del weights, typed
    torch.cuda.empty_cache()
