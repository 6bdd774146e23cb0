"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (per element): matmul outputs and combined outputs within
|gpu - oracle| / max(1, |oracle|) <= 2e-5; router ids and the id map bit
exact; renormalised gates within 2e-6; Direct and Grouped bit identical on
every shape, and both equal to the CPU evaluation of the documented f32
reduction order bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from expert_id_matmul_amd import binding as B
from expert_id_matmul_amd import workloads as W

from helpers import (GATE_TOL, GUARD, assert_close, canonical_matmul_id, check_guarded,
                     ids_to_dev, poisoned_output, to_dev, u32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _wl(name, dtype, m, n, k, top_k, n_experts, stride=None, layout=W.LAYOUT_SHARED,
        mult=W.IDS_DISTINCT, seed=7, ids_kind="random"):
    size = W.DTYPE_SIZE[dtype]
    return W.Workload(name, dtype, m, n, k, top_k, n_experts, stride or n * k * size, layout, mult,
                      seed, 0.5 if dtype == W.DT_F32 else 0.05, ids_kind, "softmax")


# small cases: several tiles and rounds plus ragged tails in n, k and rows
SMALL = [
    W.WORKLOADS["tiny"],
    # the page's test_shape: bf16, 9 tokens, n=11, k=37, top-6 of 8, padded 832-byte stride
    _wl("page_test_shape", W.DT_BF16, 9, 11, 37, 6, 8, stride=832, seed=11),
    # the page's A-B-A case: f32 n=5 k=7 top-3 of 4, 152-byte stride
    _wl("page_aba", W.DT_F32, 3, 5, 7, 3, 4, stride=152, seed=12),
] + [
    # the page's injected-failure shapes: f32, 5 experts, top-3
    _wl(f"page_inject_m{m}", W.DT_F32, m, n, k, 3, 5, seed=100 + m)
    for (m, n, k) in [(13, 31, 47), (14, 33, 49), (15, 35, 51), (16, 37, 53), (17, 39, 55), (18, 41, 57)]
] + [
    _wl(f"mix_{W.DTYPE_NAME[dt]}_{'slot' if lay else 'shared'}", dt, 37, 70, 300, 3, 9,
        stride=70 * 300 * W.DTYPE_SIZE[dt] + 64, layout=lay, seed=20 + dt * 2 + lay)
    for dt in (W.DT_F32, W.DT_F16, W.DT_BF16) for lay in (W.LAYOUT_SHARED, W.LAYOUT_SLOTTED)
] + [
    _wl("vec_bf16", W.DT_BF16, 33, 96, 512, 4, 16, seed=30),
    _wl("vec_f16_slot_tail", W.DT_F16, 20, 64, 264, 8, 16, layout=W.LAYOUT_SLOTTED, seed=31),
    _wl("vec_f32", W.DT_F32, 40, 72, 392, 2, 6, seed=32),
    _wl("k_below_granule", W.DT_BF16, 5, 9, 5, 2, 3, seed=33),
    _wl("n1_k1", W.DT_F32, 4, 1, 1, 2, 3, seed=34),
    _wl("one_expert_top1", W.DT_F16, 17, 40, 96, 1, 1, seed=35),
    _wl("m1_decode_like", W.DT_BF16, 1, 136, 1024, 8, 64, seed=36),
    # aligned rows too long for the Direct block to stage the activation row
    # in LDS: Direct reads it per slice from memory
    _wl("vec_bf16_long_k", W.DT_BF16, 3, 40, 4224, 4, 8, seed=38),
    _wl("may_repeat", W.DT_BF16, 12, 48, 256, 5, 3, mult=W.IDS_MAY_REPEAT, seed=37, ids_kind="repeat"),
    # k a whole number of 128-element rounds: Grouped streams the rounds of
    # consecutive jobs; these give blocks several jobs each, in odd and even
    # numbers, with a ragged last column tile
    _wl("stream_bf16_jobs", W.DT_BF16, 256, 1000, 512, 8, 16, seed=60),
    _wl("stream_f16_slot", W.DT_F16, 150, 700, 256, 6, 10, layout=W.LAYOUT_SLOTTED, seed=61),
    _wl("stream_f32", W.DT_F32, 128, 2000, 256, 4, 8, seed=62),
    # an odd number of rounds (3 and 5): jobs alternate between starting on a
    # step and one round later, one step holding two jobs' rounds; blocks of
    # 4 or 5 jobs, 1 or 2 and 3, last row tiles with and without
    # rows in the upper half of the tile (k = 384, 640)
    _wl("stream_odd_bf16_jobs", W.DT_BF16, 256, 1000, 384, 8, 16, seed=63),
    _wl("stream_odd_bf16_five", W.DT_BF16, 300, 1000, 640, 8, 16, seed=64),
    _wl("stream_odd_f16_slot", W.DT_F16, 150, 700, 384, 6, 10, layout=W.LAYOUT_SLOTTED, seed=65),
    _wl("stream_odd_f32", W.DT_F32, 150, 2000, 384, 4, 8, seed=66),
    # k past the last whole round (rows still whole 16-byte pieces): the last
    # round's pieces past k enter as zeros; even and odd round counts, f32
    # granules half inside k (k = 300, 132)
    _wl("stream_tail_bf16_jobs", W.DT_BF16, 256, 1000, 1000, 8, 16, seed=67),
    _wl("stream_tail_odd_bf16", W.DT_BF16, 300, 1000, 1064, 8, 16, seed=68),
    _wl("stream_tail_f16_slot", W.DT_F16, 150, 700, 2880, 6, 10, layout=W.LAYOUT_SLOTTED, seed=69),
    _wl("stream_tail_f32", W.DT_F32, 150, 2000, 300, 4, 8, seed=70),
    _wl("stream_tail_f32_two_rounds", W.DT_F32, 128, 2000, 132, 4, 8, seed=71),
]


def _ids(wl):
    if wl.ids_kind == "repeat":
        rng = np.random.default_rng(wl.seed)
        return rng.integers(0, wl.n_experts, size=(wl.m, wl.top_k)).astype(np.uint32)
    return W.ids(wl)


def run_matmul(lib, wl, wdev, x, ids, route, allow_nan=False):
    out = poisoned_output(wl.routed_rows * wl.n)
    scratch = None
    if route == B.GROUPED:
        need = lib.query(B.shape_of(wl), B.GROUPED).scratch_bytes
        scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    taken = lib.matmul_id(B.shape_of(wl), route, wdev, to_dev(x), ids_to_dev(ids), out, scratch,
                          weight_bytes=wl.weight_bytes)
    assert taken == route
    torch.cuda.synchronize()
    return check_guarded(out, wl.routed_rows * wl.n, allow_nan).reshape(wl.routed_rows, wl.n)


def _oracle_y(wl, wb, x, ids):
    return oracle.matmul_id(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout,
                            wb, x, ids)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_matmul_small_parity_and_bit_identity(lib, wl):
    print(f"[case] matmul {wl.name}", flush=True)
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = _ids(wl)
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32)), "Direct and Grouped differ"
    assert_close(yd, _oracle_y(wl, wb, x, ids), what=wl.name)
    canon = canonical_matmul_id(wl, wb, x, ids)
    assert np.array_equal(yd.view(np.uint32), canon.view(np.uint32)), "not the documented order"


@pytest.mark.parametrize("profile", ["balanced", "skewed", "repeat"])
def test_bit_identity_on_the_pages_calibration_inputs(lib, profile):
    """Adversarial activations and the balanced / maximally skewed / repeating
    id profiles of the page's calibration (fn calibration_buffers)."""
    print(f"[case] calibration profile {profile}", flush=True)
    mult = W.IDS_MAY_REPEAT if profile == "repeat" else W.IDS_DISTINCT
    wl = _wl("calib", W.DT_BF16, 64, 100, 640, 6, 24, mult=mult, seed=40)
    wb = W.weight_bytes(wl)
    x = W.adversarial_activations(wl.m, wl.k)
    ids = W.profile_ids(wl.m, wl.top_k, wl.n_experts, profile)
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32))
    assert_close(yd, _oracle_y(wl, wb, x, ids), what=profile)
    assert np.array_equal(yd.view(np.uint32), canonical_matmul_id(wl, wb, x, ids).view(np.uint32))


# Special operand values: each route takes its multiply-adds on a different
# unit (Grouped on the matrix core, Direct as vector fmas), so the classes
# where two implementations of an fma could differ are planted on purpose.
_FINITE_F32 = np.array([0x00000001, 0x807fffff, 0x00400000, 0x80000000, 0x00000000, 0x7f7fffff, 0x00800000,
                        0x3f800001], dtype=np.uint32)
_NONFINITE_F32 = np.array([0x7f800000, 0xff800000, 0x7fc00001, 0xffc12345], dtype=np.uint32)
_FINITE_16 = {
    W.DT_F16: np.array([0x0001, 0x83ff, 0x0200, 0x8000, 0x0000, 0x7bff, 0x0400], dtype=np.uint16),
    W.DT_BF16: np.array([0x0001, 0x807f, 0x0040, 0x8000, 0x0000, 0x7f7f, 0x0080], dtype=np.uint16),
}
_NONFINITE_16 = {
    W.DT_F16: np.array([0x7c00, 0xfc00, 0x7e01, 0xfe35], dtype=np.uint16),
    W.DT_BF16: np.array([0x7f80, 0xff80, 0x7fc1, 0xffc5], dtype=np.uint16),
}


def _plant(rng, bits: np.ndarray, special: np.ndarray, frac: float) -> np.ndarray:
    bits = bits.copy()
    where = rng.random(bits.shape) < frac
    bits[where] = special[rng.integers(0, len(special), int(where.sum()))]
    return bits


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_F16, W.DT_BF16], ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("k", [512, 384, 1064, 300], ids=["streamed", "streamed_odd", "streamed_tail", "k300"])
def test_bit_identity_with_special_values(lib, dtype, k):
    """Subnormal, signed-zero, infinite, NaN and extreme weights and activations:
    Direct and Grouped give the same bits (NaN for NaN), and so does the CPU
    evaluation of the documented order."""
    print(f"[case] special values dtype={dtype} k={k}", flush=True)
    wl = _wl("special", dtype, 7, 40, k, 3, 5, seed=90 + dtype)
    rng = np.random.default_rng(900 + 10 * dtype + (k % 7))
    wb = W.weight_bytes(wl)
    # finite specials often, infinities and NaNs rarely (most outputs stay finite)
    if dtype == W.DT_F32:
        wbits = _plant(rng, wb.view(np.uint32), _FINITE_F32, 0.05)
        wb = _plant(rng, wbits, _NONFINITE_F32, 0.0005).view(np.uint8)
    else:
        wbits = _plant(rng, wb.view(np.uint16), _FINITE_16[dtype], 0.05)
        wb = _plant(rng, wbits, _NONFINITE_16[dtype], 0.0005).view(np.uint8)
    xbits = _plant(rng, W.activations(wl).view(np.uint32), _FINITE_F32, 0.05)
    x = _plant(rng, xbits, _NONFINITE_F32, 0.0005).view(np.float32)
    ids = _ids(wl)
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT, allow_nan=True)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED, allow_nan=True)
    canon = canonical_matmul_id(wl, wb, x, ids)

    def same(a, b):
        both_nan = np.isnan(a) & np.isnan(b)
        return bool(np.all(both_nan | (a.view(np.uint32) == b.view(np.uint32))))

    assert np.isnan(yd).any() and np.isfinite(yd).any(), "the planted values should reach the outputs"
    assert same(yd, yg), "Direct and Grouped differ"
    assert same(yd, canon), "not the documented order"


def test_modular_fill_weights(lib):
    """The page's deterministic f32 weight fill ((19 i + 37 seed) mod 257 - 128) / 263."""
    wl = _wl("modfill", W.DT_F32, 13, 31, 47, 3, 5, seed=101)
    wb = W.modular_fill(wl.n_experts * wl.n * wl.k, 101).view(np.uint8)
    x = W.adversarial_activations(wl.m, wl.k)
    ids = W.profile_ids(wl.m, 3, 5, "balanced")
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32))
    assert_close(yd, _oracle_y(wl, wb, x, ids))


@pytest.mark.parametrize("m,n,k", [(10, 40, 200), (200, 640, 512), (200, 640, 384), (200, 640, 1000)],
                         ids=["short", "streamed", "streamed_odd", "streamed_tail"])
def test_ids_naming_no_expert_give_nan_rows_in_both_routes(lib, m, n, k):
    print(f"[case] bad ids m={m} n={n} k={k}", flush=True)
    wl = _wl("bad_ids", W.DT_BF16, m, n, k, 3, 6, seed=50)
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = W.ids(wl).copy()
    ids[2, 1] = 6
    ids[7, 0] = 0xFFFFFFFF
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT, allow_nan=True)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED, allow_nan=True)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32))
    bad = [2 * 3 + 1, 7 * 3 + 0]
    assert np.isnan(yd[bad]).all()
    assert np.isfinite(np.delete(yd, bad, axis=0)).all()
    assert_close(yd, _oracle_y(wl, wb, x, ids))


def test_row_and_slot_permutation_permute_outputs_bitwise(lib):
    wl = _wl("perm", W.DT_BF16, 24, 64, 384, 4, 12, seed=51)
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = W.ids(wl)
    wdev = to_dev(wb)
    perm = np.random.default_rng(1).permutation(wl.m)
    for route in (B.DIRECT, B.GROUPED):
        y = run_matmul(lib, wl, wdev, x, ids, route).reshape(wl.m, wl.top_k, wl.n)
        yp = run_matmul(lib, wl, wdev, x[perm], ids[perm], route).reshape(wl.m, wl.top_k, wl.n)
        assert np.array_equal(yp.view(np.uint32), y[perm].view(np.uint32))
        sp = np.array([3, 1, 0, 2])
        ys = run_matmul(lib, wl, wdev, x, ids[:, sp], route).reshape(wl.m, wl.top_k, wl.n)
        assert np.array_equal(ys.view(np.uint32), y[:, sp].view(np.uint32))


# ------------------------------------------------------------------ router
@pytest.mark.parametrize("m,n_experts,top_k,with_bias", [
    (300, 256, 8, True), (77, 8, 2, True), (64, 64, 6, False), (50, 100, 7, True),
    (9, 2048, 8, True), (33, 128, 1, True), (5, 16, 16, True), (2, 1, 1, False),
])
def test_router_ids_exact_and_gates_close(lib, m, n_experts, top_k, with_bias):
    print(f"[case] router m={m} E={n_experts} top_k={top_k}", flush=True)
    logits = W.random_f32((m, n_experts), 60, m, n_experts)
    bias = (W.random_f32((n_experts,), 61, n_experts) * 0.1).astype(np.float32) if with_bias else None
    ids_o, gates_o, _, _ = oracle.route(logits, bias, top_k)
    ids = torch.empty((m, top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((m, top_k), dtype=torch.float32, device="cuda")
    lib.route_topk(to_dev(logits), None if bias is None else to_dev(bias), top_k, ids, gates)
    torch.cuda.synchronize()
    assert np.array_equal(u32(ids), ids_o)
    g = gates.cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(g - gates_o) / gates_o)) <= GATE_TOL


def test_router_ties_and_raw_scores(lib):
    logits = np.zeros((4, 32), np.float32)
    logits[1, 7] = logits[1, 30] = 2.0
    ids = torch.empty((4, 5), dtype=torch.int32, device="cuda")
    gates = torch.empty((4, 5), dtype=torch.float32, device="cuda")
    lib.route_topk(to_dev(logits), None, 5, ids, gates, renormalize=False)
    torch.cuda.synchronize()
    got = u32(ids)
    assert list(got[0]) == [0, 1, 2, 3, 4]
    assert list(got[1]) == [7, 30, 0, 1, 2]
    ids_o, g_o, _, _ = oracle.route(logits, None, 5, renormalize=False)
    assert np.array_equal(got, ids_o)
    assert np.array_equal(gates.cpu().numpy().astype(np.float64), g_o)


# ------------------------------------------------------------------ map
# Up to 16384 routed rows (and at most 2^24 ids read over all keys) the map is
# one launch with a block per key; above, a histogram pass and a scatter pass.
# "rows_16384" fills every chunk of the one-launch form; "rows_16388" and
# "experts_2048" are just past its two limits.
@pytest.mark.parametrize("case", ["balanced", "skewed", "repeat", "random", "invalid", "large",
                                  "rows_16384", "rows_16388", "experts_2048"])
def test_map_is_exact(lib, case):
    print(f"[case] map {case}", flush=True)
    if case in ("balanced", "skewed", "repeat"):
        m, top_k, E = 512, 8, 128
        ids = W.profile_ids(m, top_k, E, case)
    elif case == "large":
        m, top_k, E = 2048, 8, 256
        logits = W.random_f32((m, E), 70)
        ids = oracle.route(logits, None, top_k)[0]
    elif case in ("rows_16384", "rows_16388", "experts_2048"):
        m, top_k, E = {"rows_16384": (16384, 1, 8), "rows_16388": (4097, 4, 64),
                       "experts_2048": (1024, 16, 2048)}[case]
        ids = np.random.default_rng(72).integers(0, E, size=(m, top_k)).astype(np.uint32)
        ids[7, 0] = E + 3  # one id naming no expert
    else:
        m, top_k, E = 300, 5, 37
        ids = np.random.default_rng(71).integers(0, E, size=(m, top_k)).astype(np.uint32)
        if case == "invalid":
            ids[5, 1] = E
            ids[100, 4] = 0xFFFFFFFF
            ids[299, 0] = 1000
    counts = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 2, dtype=torch.int32, device="cuda")
    rows = torch.empty(m * top_k, dtype=torch.int32, device="cuda")
    scratch = torch.empty(lib.map_scratch_bytes(m, top_k, E), dtype=torch.uint8, device="cuda")
    lib.map(ids_to_dev(ids), E, counts, offsets, rows, scratch)
    torch.cuda.synchronize()
    c_o, o_o, r_o = oracle.id_map(ids, E)
    assert np.array_equal(u32(counts), c_o)
    assert np.array_equal(u32(offsets), o_o)
    assert np.array_equal(u32(rows), r_o)


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("m,top_k,n", [(7, 3, 33), (64, 8, 256), (1, 8, 1536), (5, 1, 2)])
def test_combine_parity(lib, m, top_k, n):
    y = W.random_f32((m * top_k, n), 80, m, n)
    g = np.abs(W.random_f32((m, top_k), 81, m))
    out = poisoned_output(m * n)
    lib.combine(to_dev(y), to_dev(g), out)
    torch.cuda.synchronize()
    got = check_guarded(out, m * n).reshape(m, n)
    assert_close(got, oracle.combine(y.astype(np.float64), g.astype(np.float64), top_k))


def test_combine_one_hot_gates_copy_rows_bitwise(lib):
    m, top_k, n = 6, 4, 40
    y = W.random_f32((m * top_k, n), 82)
    for j in range(top_k):
        g = np.zeros((m, top_k), np.float32)
        g[:, j] = 1.0
        out = torch.empty((m, n), dtype=torch.float32, device="cuda")
        lib.combine(to_dev(y), to_dev(g), out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), y.reshape(m, top_k, n)[:, j].view(np.uint32))


# ------------------------------------------------------------------ whole path
@pytest.mark.parametrize("route", [B.DIRECT, B.GROUPED, B.AUTO])
def test_moe_forward_small_down_projection(lib, route):
    """Slotted input, f16 experts, sigmoid + bias routing, gate-weighted sum."""
    wl = W.small("down_proj", m=48, n=96, k=200, n_experts=32, top_k=4)
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    logits = W.router_logits(wl)
    bias = W.router_bias(wl)
    ids_o, gates_o, _, _ = oracle.route(logits, bias, wl.top_k)
    y_o = _oracle_y(wl, wb, x, ids_o)
    out_o = oracle.combine(y_o, gates_o, wl.top_k)
    dev = lambda a: to_dev(a)
    ids = torch.empty((wl.m, wl.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((wl.m, wl.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    out = poisoned_output(wl.m * wl.n)
    need = lib.query(B.shape_of(wl), B.GROUPED).scratch_bytes
    scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    taken = lib.moe_forward(B.shape_of(wl), route, dev(wb), dev(x), dev(logits), dev(bias), ids,
                            gates, y, out, scratch, weight_bytes=wl.weight_bytes)
    torch.cuda.synchronize()
    assert taken in (B.DIRECT, B.GROUPED)
    assert np.array_equal(u32(ids), ids_o)
    assert_close(y.cpu().numpy(), y_o, what="y")
    assert_close(check_guarded(out, wl.m * wl.n).reshape(wl.m, wl.n), out_o, what="out")


@pytest.mark.parametrize("dtype,m,n,k,top_k,n_experts,layout", [
    (W.DT_BF16, 3, 200, 1000, 8, 256, W.LAYOUT_SHARED),    # decode-like, ragged n, k tail
    (W.DT_F32, 2, 37, 64, 5, 300, W.LAYOUT_SLOTTED),       # > 256 experts, k below one round
    (W.DT_F16, 4, 64, 256, 16, 64, W.LAYOUT_SHARED),       # 16 slots per token
    (W.DT_BF16, 5, 48, 384, 1, 7, W.LAYOUT_SLOTTED),       # one slot
    (W.DT_BF16, 2, 96, 512, 8, 1000, W.LAYOUT_SHARED),     # > 256 experts, staged activation row
    (W.DT_BF16, 1, 24, 8320, 2, 16, W.LAYOUT_SHARED),      # row too long to stage: read from memory
    # 8 slots and at most 256 experts: the first 256 threads score the experts
    # (those past n_experts as empty entries) while the others copy the row
    (W.DT_F16, 1, 300, 2048, 8, 130, W.LAYOUT_SHARED),
    (W.DT_BF16, 2, 100, 512, 8, 200, W.LAYOUT_SLOTTED),    # the same split with no row to copy
    # staged row with a partial last round and too many experts to split
    # the roles (512 threads, 320 router entries)
    (W.DT_F16, 2, 70, 1000, 8, 300, W.LAYOUT_SHARED),
], ids=["bf16_decode_like", "f32_many_experts", "f16_top16", "bf16_top1", "bf16_many_experts_shared",
        "bf16_long_k_shared", "f16_split_roles_130_experts", "bf16_split_roles_slotted",
        "f16_staged_tail_shared_roles"])
def test_moe_forward_direct_matches_the_three_calls_bitwise(lib, dtype, m, n, k, top_k, n_experts, layout):
    """With the Direct route the whole path runs as one kernel; its ids, gates,
    y and out must be the bits of route_topk -> matmul_id -> combine."""
    print(f"[case] fused moe_forward dtype={dtype} m={m} n={n} k={k} top_k={top_k} E={n_experts}", flush=True)
    _fused_vs_three_calls(lib, _wl("fused", dtype, m, n, k, top_k, n_experts, layout=layout, seed=70 + top_k),
                          with_bias=True, renormalize=True)


def test_moe_forward_direct_without_bias_or_renormalisation(lib):
    print("[case] fused moe_forward without bias, raw gates", flush=True)
    _fused_vs_three_calls(lib, _wl("fused_plain", W.DT_BF16, 3, 40, 256, 4, 32, seed=79),
                          with_bias=False, renormalize=False)


def _fused_vs_three_calls(lib, wl, with_bias, renormalize):
    m, n, top_k = wl.m, wl.n, wl.top_k
    wl = wl.with_(ids_kind="logits")
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    logits = W.router_logits(wl)
    bias = W.router_bias(wl) if with_bias else None
    bias_dev = to_dev(bias) if with_bias else None
    shape = B.shape_of(wl)
    wdev = to_dev(wb)

    def bufs():
        return (torch.empty((m, top_k), dtype=torch.int32, device="cuda"),
                torch.empty((m, top_k), dtype=torch.float32, device="cuda"),
                poisoned_output(wl.routed_rows * n), poisoned_output(m * n))

    ids_f, gates_f, y_f, out_f = bufs()
    taken = lib.moe_forward(shape, B.DIRECT, wdev, to_dev(x), to_dev(logits), bias_dev, ids_f, gates_f,
                            y_f, out_f, None, renormalize=renormalize, weight_bytes=wl.weight_bytes)
    assert taken == B.DIRECT
    ids_s, gates_s, y_s, out_s = bufs()
    lib.route_topk(to_dev(logits), bias_dev, top_k, ids_s, gates_s, renormalize=renormalize)
    lib.matmul_id(shape, B.DIRECT, wdev, to_dev(x), ids_s, y_s, None, weight_bytes=wl.weight_bytes)
    lib.combine(y_s[:wl.routed_rows * n].view(wl.routed_rows, n), gates_s, out_s[:m * n].view(m, n))
    torch.cuda.synchronize()
    assert torch.equal(ids_f, ids_s)
    assert torch.equal(gates_f.view(torch.int32), gates_s.view(torch.int32))
    yf = check_guarded(y_f, wl.routed_rows * n)
    assert np.array_equal(yf.view(np.uint32), check_guarded(y_s, wl.routed_rows * n).view(np.uint32))
    of = check_guarded(out_f, m * n)
    assert np.array_equal(of.view(np.uint32), check_guarded(out_s, m * n).view(np.uint32))
    ids_o, gates_o, _, _ = oracle.route(logits, bias, top_k, renormalize=renormalize)
    assert np.array_equal(u32(ids_f), ids_o)
    y_o = _oracle_y(wl, wb, x, ids_o)
    assert_close(yf.reshape(wl.routed_rows, n), y_o, what="fused y")
    assert_close(of.reshape(m, n), oracle.combine(y_o, gates_o, top_k), what="fused out")


# ------------------------------------------------------------------ id validation
def _first_bad(ids: np.ndarray, n_experts: int, distinct: bool) -> int:
    """Brute force: the smallest flat index whose id names no expert or repeats
    an earlier slot of its token."""
    m, top_k = ids.shape
    for t in range(m):
        for s in range(top_k):
            if ids[t, s] >= n_experts or (distinct and ids[t, s] in ids[t, :s]):
                return t * top_k + s
    return -1


@pytest.mark.parametrize("case", ["good", "out_of_range", "repeat", "repeat_allowed", "several", "max_id"])
def test_validate_ids_finds_the_first_bad_entry(lib, case):
    print(f"[case] validate ids {case}", flush=True)
    rng = np.random.default_rng(90)
    m, top_k, E = 300, 6, 40
    ids = np.stack([rng.permutation(E)[:top_k] for _ in range(m)]).astype(np.uint32)
    distinct = case != "repeat_allowed"
    if case == "out_of_range":
        ids[123, 4] = E
    elif case in ("repeat", "repeat_allowed"):
        ids[77, 5] = ids[77, 2]
    elif case == "several":
        ids[200, 1] = 0xFFFFFFFF
        ids[150, 3] = ids[150, 0]
        ids[299, 5] = E + 7
    elif case == "max_id":
        ids[0, 0] = E - 1
        ids[0, 1:] = np.arange(top_k - 1)
    want = _first_bad(ids, E, distinct)
    got = lib.validate_ids(ids_to_dev(ids), E, 0 if distinct else 1)
    assert got == want
    if case in ("good", "repeat_allowed", "max_id"):
        assert got == -1


# ------------------------------------------------------------------ random shapes
def _random_shape(seed: int):
    """A seeded small shape around the kernels' boundaries: k near multiples
    of 128 and 256 (streamed or masked Grouped, staged or per-slice Direct
    activations), ragged n, up to 300 experts and 16 slots, both layouts,
    padded expert strides."""
    rng = np.random.default_rng(seed)
    dtype = int(rng.integers(0, 3))
    size = W.DTYPE_SIZE[dtype]
    k = int(rng.choice([1, 7, 64, 127, 128, 129, 255, 256, 257, 384, 512, 640, 768, 1024, 1032]))
    n = int(rng.integers(1, 300))
    n_experts = int(rng.choice([1, 2, 5, 16, 64, 300]))
    top_k = int(rng.integers(1, min(n_experts, 16) + 1))
    m = int(rng.integers(1, 90))
    layout = int(rng.integers(0, 2))
    mult = int(rng.integers(0, 2))
    pad = int(rng.choice([0, 0, 16, 48, 2]))
    stride = n * k * size + pad * size
    kind = "repeat" if mult == W.IDS_MAY_REPEAT else "random"
    return _wl(f"rand{seed}", dtype, m, n, k, top_k, n_experts, stride=stride, layout=layout, mult=mult,
               seed=200 + seed, ids_kind=kind)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_parity_and_bit_identity(lib, seed):
    wl = _random_shape(seed)
    print(f"[case] random shape {seed}: dtype={wl.dtype} m={wl.m} n={wl.n} k={wl.k} top_k={wl.top_k} "
          f"E={wl.n_experts} layout={wl.layout} mult={wl.multiplicity} stride={wl.stride}", flush=True)
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = _ids(wl)
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32)), "Direct and Grouped differ"
    assert_close(yd, _oracle_y(wl, wb, x, ids), what=wl.name)
    assert np.array_equal(yd.view(np.uint32), canonical_matmul_id(wl, wb, x, ids).view(np.uint32))


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_fused_step_matches_the_three_calls(lib, seed):
    """The one-kernel route -> Direct -> combine step on seeded small shapes
    (staged and per-slice activations, 1 to 16 slots, up to 300 experts,
    with and without bias and renormalisation)."""
    rng = np.random.default_rng(500 + seed)
    dtype = int(rng.integers(0, 3))
    k = int(rng.choice([64, 128, 200, 256, 1000, 2048, 4096, 4104]))
    n = int(rng.integers(1, 200))
    n_experts = int(rng.choice([1, 8, 64, 256, 300]))
    top_k = int(rng.integers(1, min(n_experts, 16) + 1))
    m = int(rng.integers(1, 6))
    layout = int(rng.integers(0, 2))
    with_bias, renorm = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    print(f"[case] random fused {seed}: dtype={dtype} m={m} n={n} k={k} top_k={top_k} E={n_experts} "
          f"layout={layout} bias={with_bias} renorm={renorm}", flush=True)
    _fused_vs_three_calls(lib, _wl(f"rfused{seed}", dtype, m, n, k, top_k, n_experts, layout=layout,
                                   seed=600 + seed), with_bias=with_bias, renormalize=renorm)


def test_router_sigmoid_bits_over_ten_million_logits(lib):
    """gate = sigma(logit) when one expert is picked without renormalising: the
    GPU's f32 sigma equals the oracle's bit for bit over 10^7 logits spanning
    [-88, 88] (a uniform grid, random values, and dense runs where sigma
    saturates to 1 in f32 and where it falls into the subnormal range)."""
    rng = np.random.default_rng(97)
    parts = [np.linspace(-88.0, 88.0, 6_000_000, dtype=np.float64).astype(np.float32),
             rng.uniform(-88.0, 88.0, 2_000_000).astype(np.float32),
             rng.uniform(15.0, 18.5, 800_000).astype(np.float32),     # sigma -> 1 - 2^-24 .. 1
             rng.uniform(-88.0, -80.0, 800_000).astype(np.float32),   # sigma below 2^-115, subnormal f32 tail
             rng.uniform(-1e-3, 1e-3, 399_992).astype(np.float32),
             np.array([0.0, -0.0, 88.0, -88.0, 1e-30, -1e-30, 17.328680, -87.33655], dtype=np.float32)]
    logits = np.concatenate(parts).reshape(-1, 1)
    m = logits.shape[0]
    assert m >= 10_000_000
    print(f"[case] sigmoid sweep m={m}", flush=True)
    ids = torch.empty((m, 1), dtype=torch.int32, device="cuda")
    gates = torch.empty((m, 1), dtype=torch.float32, device="cuda")
    lib.route_topk(to_dev(logits), None, 1, ids, gates, renormalize=False)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == 0).all()
    _, _, sigma, _ = oracle.route(logits, None, 1, renormalize=False)
    g = gates.cpu().numpy().view(np.uint32).reshape(-1)
    o = sigma.view(np.uint32).reshape(-1)
    bad = np.flatnonzero(g != o)
    assert bad.size == 0, f"{bad.size} sigma values differ, e.g. logit {logits.reshape(-1)[bad[:3]]}"


# ------------------------------------------------------- uneven expert loads
def _zipf_ids(m: int, top_k: int, n_experts: int, seed: int, a: float = 1.2) -> np.ndarray:
    """Distinct ids per token drawn with P(e) proportional to 1/(e+1)^a: a few
    experts with hundreds of rows, many with 1 to 48, some with none."""
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, n_experts + 1) ** a
    p /= p.sum()
    return np.stack([rng.choice(n_experts, size=top_k, replace=False, p=p) for _ in range(m)]).astype(np.uint32)


@pytest.mark.parametrize("dtype,k", [(W.DT_BF16, 384), (W.DT_F16, 1000), (W.DT_BF16, 2048)],
                         ids=["bf16_k384", "f16_k1000", "bf16_k2048"])
def test_uneven_expert_loads_bit_identity(lib, dtype, k):
    """Expert row counts from a heavy-tailed draw, over 16 column tiles: the
    Grouped kernel cuts its job list into XCD shares by cost (a job of at
    most 16 rows costs half), so the cuts land inside buckets, between and
    among their short last tiles.  Every output must still be computed once,
    equal to Direct's bits and to the documented order, and within the bar of
    the oracle (k = 384 and 1000 run the build with accumulators in the
    accumulation registers, k = 2048 the other)."""
    from helpers import host_threads
    wl = _wl(f"uneven_{dtype}_{k}", dtype, 600, 1000, k, 4, 96, seed=90 + k % 7)
    print(f"[case] uneven expert loads dtype={dtype} k={k}", flush=True)
    wb = W.weight_bytes(wl)
    x = W.activations(wl)
    ids = _zipf_ids(wl.m, wl.top_k, wl.n_experts, seed=k)
    counts = np.bincount(ids.reshape(-1), minlength=wl.n_experts)
    assert counts.max() > 256 and ((counts > 0) & (counts % 32 <= 16) & (counts % 32 > 0)).sum() > 10
    wdev = to_dev(wb)
    yd = run_matmul(lib, wl, wdev, x, ids, B.DIRECT)
    yg = run_matmul(lib, wl, wdev, x, ids, B.GROUPED)
    assert np.array_equal(yd.view(np.uint32), yg.view(np.uint32)), "Direct and Grouped differ"
    threads = host_threads()
    assert np.array_equal(yd.view(np.uint32), canonical_matmul_id(wl, wb, x, ids, threads=threads).view(np.uint32))
    ref = oracle.matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.n_experts, wl.stride, wl.layout, wb, x,
                                   ids, threads)
    assert_close(yd, ref, what=wl.name)
