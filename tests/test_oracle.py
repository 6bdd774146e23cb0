"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a fact fixed by the pages or by
mathematics: the pages' printed weight extents, exhaustive dtype decoding
against library conversions, numpy float64 brute force, closed forms of
the routing profiles, and invariants (identity expert, permutations,
placement independence, one-hot gates, monotone sigmoid).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from expert_id_matmul_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT = {"f32": W.DT_F32, "f16": W.DT_F16, "bf16": W.DT_BF16}


# ---------------------------------------------------------------- helpers
def to_f64_library(dtype: int, raw: np.ndarray, count: int) -> np.ndarray:
    """Decode native weights with library conversions (torch / numpy), not
    with the oracle's own decoder."""
    if dtype == W.DT_F32:
        return np.frombuffer(raw.tobytes(), np.float32, count).astype(np.float64)
    if dtype == W.DT_F16:
        return np.frombuffer(raw.tobytes(), np.float16, count).astype(np.float64)
    t = torch.frombuffer(bytearray(raw.tobytes()), dtype=torch.bfloat16, count=count)
    return t.to(torch.float64).numpy()


def brute_matmul_id(wl: W.Workload, wbytes, x, ids):
    """numpy float64: gather each routed row's expert matrix and contract."""
    size = W.DTYPE_SIZE[wl.dtype]
    mats = []
    for e in range(wl.n_experts):
        chunk = wbytes[e * wl.stride: e * wl.stride + wl.n * wl.k * size]
        mats.append(to_f64_library(wl.dtype, chunk, wl.n * wl.k).reshape(wl.n, wl.k))
    mats = np.stack(mats)
    flat = ids.reshape(-1).astype(np.int64)
    rows = np.arange(wl.routed_rows)
    xr = x.astype(np.float64)[rows if wl.layout == W.LAYOUT_SLOTTED else rows // wl.top_k]
    return np.einsum("rk,rnk->rn", xr, mats[flat])


def padded_weights(wl: W.Workload) -> np.ndarray:
    return W.weight_bytes(wl)


def run_oracle(wl, wbytes, x, ids):
    return oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride,
                            wl.layout, wbytes, x, ids)


# the pages' tail-heavy shapes (mlx-native dense_matmul_id_auto.rs tests):
# test_shape() and the injected-failure cases of fn injected_failure_case.
TAIL_SHAPES = [
    W.Workload("page_test_shape", W.DT_BF16, 9, 11, 37, 6, 8, 832, W.LAYOUT_SHARED,
               W.IDS_DISTINCT, 11, 0.02, "random", "softmax"),
    W.Workload("page_aba", W.DT_F32, 3, 5, 7, 3, 4, 152, W.LAYOUT_SHARED, W.IDS_DISTINCT, 12,
               0.1, "random", "softmax"),
] + [
    W.Workload(f"page_inject_{m}", W.DT_F32, m, n, k, 3, 5, n * k * 4, W.LAYOUT_SHARED,
               W.IDS_DISTINCT, 100 + m, 0.1, "random", "softmax")
    for (m, n, k) in [(13, 31, 47), (14, 33, 49), (15, 35, 51), (16, 37, 53), (17, 39, 55), (18, 41, 57)]
]


# ---------------------------------------------------------------- extents
def test_required_bytes_match_the_pages_printed_extents():
    with open(os.path.join(GOLDEN, "weight_extent.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert rows
    for dt, n, k, e, stride, want in rows:
        assert oracle.required_weight_bytes(DT[dt], int(n), int(k), int(e), int(stride)) == int(want)


def test_required_bytes_overflow_is_rejected():
    assert oracle.required_weight_bytes(W.DT_F32, 2**32 - 1, 2**32 - 1, 2**32 - 1, 2**63) == 0


# ---------------------------------------------------------------- widening
def test_bf16_widening_is_exact_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.widen_array(W.DT_BF16, bits)
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_f16_widening_is_exact_for_every_pattern_including_subnormals():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.widen_array(W.DT_F16, bits)
    lib = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))
    # the subnormal range really is exercised
    assert (np.abs(lib[(bits & 0x7C00) == 0]) > 0).sum() == 2 * 1023


def test_f32_widening_is_identity():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 1e-40, 3.4e38, np.inf], dtype=np.float32)
    for v in vals:
        assert oracle.widen(W.DT_F32, v.tobytes()) == float(v)


# ---------------------------------------------------------------- matmul_id
@pytest.mark.parametrize("wl", [W.WORKLOADS["tiny"]] + TAIL_SHAPES, ids=lambda w: w.name)
def test_matmul_id_equals_numpy_brute_force(wl):
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    y = run_oracle(wl, wb, x, ids)
    ref = brute_matmul_id(wl, wb, x, ids)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_F16, W.DT_BF16])
@pytest.mark.parametrize("layout", [W.LAYOUT_SHARED, W.LAYOUT_SLOTTED])
def test_matmul_id_brute_force_every_dtype_and_layout(dtype, layout):
    wl = W.Workload("mix", dtype, 5, 19, 23, 3, 6, 19 * 23 * W.DTYPE_SIZE[dtype] + 2 * W.DTYPE_SIZE[dtype],
                    layout, W.IDS_DISTINCT, 21 + dtype + 3 * layout, 0.5, "random", "softmax")
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    np.testing.assert_allclose(run_oracle(wl, wb, x, ids), brute_matmul_id(wl, wb, x, ids),
                               rtol=1e-12, atol=1e-12)


def test_top1_single_expert_reduces_to_a_plain_matmul():
    wl = W.Workload("top1", W.DT_BF16, 7, 24, 40, 1, 3, 24 * 40 * 2, W.LAYOUT_SHARED,
                    W.IDS_DISTINCT, 31, 0.3, "random", "softmax")
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = np.full((wl.m, 1), 2, dtype=np.uint32)
    w2 = to_f64_library(wl.dtype, wb[2 * wl.stride:], wl.n * wl.k).reshape(wl.n, wl.k)
    np.testing.assert_allclose(run_oracle(wl, wb, x, ids), x.astype(np.float64) @ w2.T,
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_F16, W.DT_BF16])
def test_identity_expert_returns_its_input_exactly(dtype):
    n = k = 33
    eye = torch.eye(n, dtype={0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[dtype])
    raw = eye.contiguous().view(torch.uint8).numpy().reshape(-1)
    wb = np.concatenate([raw, raw])  # two identity experts
    x = W.random_f32((4, k), 41, dtype)
    ids = np.array([[1, 0]] * 4, dtype=np.uint32)
    y = oracle.matmul_id(dtype, 4, n, k, 2, 2, raw.size, W.LAYOUT_SHARED, wb, x, ids)
    assert np.array_equal(y, np.repeat(x.astype(np.float64), 2, axis=0))


def test_row_permutation_permutes_outputs_exactly():
    wl = TAIL_SHAPES[2]
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    y = run_oracle(wl, wb, x, ids).reshape(wl.m, wl.top_k, wl.n)
    perm = np.random.default_rng(0).permutation(wl.m)
    yp = run_oracle(wl, wb, x[perm], ids[perm]).reshape(wl.m, wl.top_k, wl.n)
    assert np.array_equal(yp, y[perm])
    # slot permutation inside each token permutes the routed rows too
    sp = np.array([2, 0, 1])
    ys = run_oracle(wl, wb, x, ids[:, sp]).reshape(wl.m, wl.top_k, wl.n)
    assert np.array_equal(ys, y[:, sp])


def test_placement_independence_index_and_stride():
    wl = TAIL_SHAPES[0]  # bf16, padded 832-byte stride
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    y = run_oracle(wl, wb, x, ids)
    # move every expert e to index E-1-e under a larger stride
    body = wl.n * wl.k * 2
    stride2 = 1000
    wb2 = np.full((wl.n_experts - 1) * stride2 + body, 0x7F, dtype=np.uint8)
    for e in range(wl.n_experts):
        d = wl.n_experts - 1 - e
        wb2[d * stride2: d * stride2 + body] = wb[e * wl.stride: e * wl.stride + body]
    y2 = oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, stride2, wl.layout,
                          wb2, x, (wl.n_experts - 1 - ids.astype(np.int64)).astype(np.uint32))
    assert np.array_equal(y, y2)


def test_spot_outputs_equal_full_outputs():
    wl = TAIL_SHAPES[3]
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    y = run_oracle(wl, wb, x, ids)
    rng = np.random.default_rng(5)
    rows = rng.integers(0, wl.routed_rows, 50)
    cols = rng.integers(0, wl.n, 50)
    got = oracle.matmul_id_at(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride,
                              wl.layout, wb, x, ids, rows, cols)
    assert np.array_equal(got, y[rows, cols])


@pytest.mark.parametrize("threads", [1, 2, 7, 64])
def test_threaded_outputs_equal_full_outputs(threads):
    """The host-thread split of the oracle (used for the CPU baseline and the
    full-size checks) computes every output with the same routine."""
    wl = TAIL_SHAPES[3]
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    y = run_oracle(wl, wb, x, ids)
    got = oracle.matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride,
                                   wl.layout, wb, x, ids, threads)
    assert np.array_equal(got.view(np.uint64), y.view(np.uint64))


def test_out_of_range_id_gives_nan_row_only():
    wl = W.WORKLOADS["tiny"]
    wb = padded_weights(wl)
    x = W.activations(wl)
    ids = W.ids(wl).copy()
    ids[1, 0] = wl.n_experts
    y = run_oracle(wl, wb, x, ids)
    assert np.isnan(y[2]).all()
    assert np.isfinite(np.delete(y, 2, axis=0)).all()


# ---------------------------------------------------------------- routing
def test_sigmoid_matches_library_expit_rounded_to_f32():
    from scipy.special import expit
    logits = np.concatenate([W.random_f32((64, 64), 7).reshape(-1) * 4,
                             np.array([0.0, -0.0, 1e-8, -1e-8, 20, -20, 88, -88, 103, -103], np.float32)])
    m = logits.size // 2
    lg = logits[: 2 * m].reshape(2, m)
    _, _, sigma, _ = oracle.route(lg, None, 1)
    want = expit(lg.astype(np.float64)).astype(np.float32)
    assert np.array_equal(sigma, want)
    _, _, s0, _ = oracle.route(np.zeros((1, 4), np.float32), None, 1)
    assert (s0 == 0.5).all()


def test_route_with_zero_bias_is_a_plain_argsort_of_logits():
    lg = W.random_f32((40, 64), 8)
    ids, gates, _, _ = oracle.route(lg, np.zeros(64, np.float32), 6)
    want = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :6]
    assert np.array_equal(ids, want.astype(np.uint32))


def test_route_matches_brute_force_full_sort_with_bias():
    from scipy.special import expit
    lg = W.random_f32((50, 256), 9)
    bias = (W.random_f32((256,), 10) * 0.05).astype(np.float32)
    ids, gates, sigma, sel = oracle.route(lg, bias, 8)
    s = expit(lg.astype(np.float64)).astype(np.float32)
    key = (s + bias).astype(np.float32)
    for t in range(lg.shape[0]):
        # sort by key descending, ties by index ascending
        order = sorted(range(256), key=lambda e: (-float(key[t, e]), e))[:8]
        assert list(ids[t]) == order
        p = s[t, order].astype(np.float64)
        np.testing.assert_allclose(gates[t], p / p.sum(), rtol=1e-15)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=1e-14)
    # bias changes the selection, not the gates' numerators
    assert not np.array_equal(ids, oracle.route(lg, None, 8)[0])


def test_route_ties_take_the_lower_index_and_ids_are_distinct():
    lg = np.zeros((3, 16), np.float32)
    lg[1, 5] = lg[1, 9] = 1.0
    ids, gates, _, _ = oracle.route(lg, None, 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert list(ids[1]) == [5, 9, 0, 1]
    np.testing.assert_allclose(gates[0], 0.25)
    for row in ids:
        assert len(set(row.tolist())) == 4


def test_route_without_renormalisation_reports_raw_scores():
    lg = W.random_f32((5, 32), 12)
    ids, g, sigma, _ = oracle.route(lg, None, 4, renormalize=False)
    assert np.array_equal(g, np.take_along_axis(sigma, ids.astype(np.int64), 1).astype(np.float64))


def test_route_rejects_non_finite_logits():
    lg = np.zeros((2, 8), np.float32)
    lg[1, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.route(lg, None, 2)


# ---------------------------------------------------------------- combine
def test_combine_one_hot_gates_select_a_row_exactly():
    y = W.random_f32((6 * 4, 10), 13).astype(np.float64)
    for j in range(4):
        g = np.zeros((6, 4))
        g[:, j] = 1.0
        out = oracle.combine(y, g, 4)
        assert np.array_equal(out, y.reshape(6, 4, 10)[:, j])


def test_combine_equals_einsum():
    y = W.random_f32((5 * 3, 7), 14).astype(np.float64)
    g = W.random_f32((5, 3), 15).astype(np.float64)
    np.testing.assert_allclose(oracle.combine(y, g, 3),
                               np.einsum("ts,tsn->tn", g, y.reshape(5, 3, 7)), rtol=1e-14)


# ---------------------------------------------------------------- id map
def test_map_balanced_and_skewed_closed_forms():
    bal = W.profile_ids(512, 8, 128, "balanced")
    c, o, r = oracle.id_map(bal, 128)
    assert (c[:128] == 32).all() and c[128] == 0
    assert np.array_equal(o[:129], np.arange(129, dtype=np.uint32) * 32) and o[129] == 4096
    skew = W.profile_ids(512, 8, 128, "skewed")
    c, o, r = oracle.id_map(skew, 128)
    assert (c[:8] == 512).all() and (c[8:] == 0).all()
    # expert s takes rows t*8 + s in token order
    assert np.array_equal(r[:512], np.arange(512, dtype=np.uint32) * 8)
    assert np.array_equal(r[512:1024], np.arange(512, dtype=np.uint32) * 8 + 1)


def test_map_is_the_stable_sort_by_expert():
    ids = np.random.default_rng(3).integers(0, 12, size=(37, 5)).astype(np.uint32)
    ids[4, 2] = 12
    ids[9, 0] = 4_000_000_000
    c, o, r = oracle.id_map(ids, 12)
    key = np.minimum(ids.reshape(-1), 12)
    assert np.array_equal(r, np.argsort(key, kind="stable").astype(np.uint32))
    assert np.array_equal(c, np.bincount(key, minlength=13).astype(np.uint32))
    assert o[0] == 0 and np.array_equal(np.diff(o.astype(np.int64)), c.astype(np.int64))
    assert c[12] == 2


# ---------------------------------------------------------------- expert FFN
def _ffn_parts(fw):
    parts = {w: fw.part(w) for w in ("gate", "up", "down")}
    raw = {w: W.weight_bytes(p) for w, p in parts.items()}
    return parts, raw


def _ffn_brute(fw, raw, x, ids, gates):
    """numpy float64 with library decoders: gather, contract, silu, contract, sum."""
    def mats(w, rows, cols):
        size = W.DTYPE_SIZE[fw.dtype]
        return np.stack([to_f64_library(fw.dtype, raw[w][e * rows * cols * size:(e + 1) * rows * cols * size],
                                        rows * cols).reshape(rows, cols) for e in range(fw.n_experts)])
    wg, wu, wd = mats("gate", fw.inter, fw.hidden), mats("up", fw.inter, fw.hidden), mats("down", fw.hidden, fw.inter)
    e = ids.reshape(-1).astype(np.int64)
    xr = x.astype(np.float64)[np.arange(fw.m * fw.top_k) // fw.top_k]
    g = np.einsum("rc,rjc->rj", xr, wg[e])
    u = np.einsum("rc,rjc->rj", xr, wu[e])
    h = g / (1.0 + np.exp(-g)) * u
    y = np.einsum("rj,rij->ri", h, wd[e])
    return (y.reshape(fw.m, fw.top_k, fw.hidden) * gates.reshape(fw.m, fw.top_k, 1)).sum(axis=1)


FFN_SMALL = [W.FfnWorkload("ffn_tiny_f32", W.DT_F32, 5, 12, 8, 2, 4, 41, 0.3),
             W.FfnWorkload("ffn_tiny_bf16", W.DT_BF16, 4, 16, 10, 3, 6, 42, 0.3),
             W.FfnWorkload("ffn_tiny_f16", W.DT_F16, 3, 9, 7, 2, 5, 43, 0.3)]


@pytest.mark.parametrize("fw", FFN_SMALL, ids=lambda f: f.name)
def test_ffn_equals_numpy_brute_force(fw):
    parts, raw = _ffn_parts(fw)
    x, logits, bias = W.ffn_inputs(fw)
    ids, gates, _, _ = oracle.route(logits, bias, fw.top_k)
    out, h = oracle.moe_ffn(fw.dtype, fw.m, fw.hidden, fw.inter, fw.top_k, fw.n_experts,
                            parts["gate"].stride, parts["down"].stride, raw["gate"], raw["up"], raw["down"],
                            x, ids, gates)
    np.testing.assert_allclose(out, _ffn_brute(fw, raw, x, ids, gates), rtol=1e-12, atol=1e-14)


def test_ffn_silu_odd_identity_zero_up_and_linearity():
    fw = FFN_SMALL[1]
    parts, raw = _ffn_parts(fw)
    x, logits, bias = W.ffn_inputs(fw)
    ids, gates, _, _ = oracle.route(logits, bias, fw.top_k)
    args = (fw.dtype, fw.m, fw.hidden, fw.inter, fw.top_k, fw.n_experts, parts["gate"].stride,
            parts["down"].stride)
    out, h = oracle.moe_ffn(*args, raw["gate"], raw["up"], raw["down"], x, ids, gates)
    # silu(v) - silu(-v) = v: negating W_gate (exact in every dtype) gives h' with h - h' = g * u,
    # and with W_up = W_gate that is g^2 >= 0 row by row
    neg = raw["gate"].copy()
    size = W.DTYPE_SIZE[fw.dtype]
    sign_byte = np.arange(neg.size) % size == size - 1
    neg[sign_byte] ^= 0x80
    _, h_pos = oracle.moe_ffn(*args, raw["gate"], raw["gate"], raw["down"], x, ids, gates)
    _, h_neg = oracle.moe_ffn(*args, neg, raw["gate"], raw["down"], x, ids, gates)
    g_direct = oracle.matmul_id(fw.dtype, fw.m, fw.inter, fw.hidden, fw.top_k, fw.n_experts,
                                parts["gate"].stride, W.LAYOUT_SHARED, raw["gate"], x, ids)
    np.testing.assert_allclose(h_pos - h_neg, g_direct * g_direct, rtol=1e-12, atol=1e-15)
    # W_up = 0 -> out = 0 exactly
    zero, _ = oracle.moe_ffn(*args, raw["gate"], np.zeros_like(raw["up"]), raw["down"], x, ids, gates)
    assert (zero == 0).all()
    # doubling W_down (exact: exponent + 1 for these magnitudes) doubles out exactly
    dbl = np.frombuffer(raw["down"].tobytes(), np.uint16).copy()
    nz = dbl & 0x7FFF != 0
    dbl[nz] += 0x80  # bf16 exponent field starts at bit 7
    out2, _ = oracle.moe_ffn(*args, raw["gate"], raw["up"], dbl.view(np.uint8), x, ids, gates)
    np.testing.assert_array_equal(out2, 2.0 * out)


def test_ffn_with_identity_down_is_the_composition_of_pinned_steps():
    """inter = hidden and W_down = I: out = combine(silu(gate.x) * up.x) from the
    already pinned matmul_id and combine."""
    fw = W.FfnWorkload("ffn_id", W.DT_F32, 4, 6, 6, 2, 3, 44, 0.5)
    parts, raw = _ffn_parts(fw)
    eye = np.tile(np.eye(6, dtype=np.float32).reshape(-1), fw.n_experts).view(np.uint8)
    x, logits, bias = W.ffn_inputs(fw)
    ids, gates, _, _ = oracle.route(logits, bias, fw.top_k)
    out, _ = oracle.moe_ffn(fw.dtype, fw.m, 6, 6, fw.top_k, fw.n_experts, parts["gate"].stride,
                            parts["down"].stride, raw["gate"], raw["up"], eye, x, ids, gates)
    mm = lambda w: oracle.matmul_id(fw.dtype, fw.m, 6, 6, fw.top_k, fw.n_experts, parts["gate"].stride,
                                    W.LAYOUT_SHARED, raw[w], x, ids)
    g, u = mm("gate"), mm("up")
    want = oracle.combine(g / (1.0 + np.exp(-g)) * u, gates, fw.top_k)
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)
