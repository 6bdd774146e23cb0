"""Seeded synthetic inputs for the expert-ID matmul workloads.

This module only draws inputs: random tensors, routing-profile ids and the
deterministic fills the pages use in their tests.  It holds none of the
method's arithmetic (no routing, no matmul, no combine), so the CPU oracle
and the HIP library can both be fed from it without sharing any code.

Random tensors are drawn with PyTorch's CPU generator, one generator per
(workload seed, tensor, index) triple, so one expert's weights can be
redrawn on their own (the oracle's spot checks at full size need only the
experts a token touched).  Half-precision weights are rounded to nearest
even from the f32 draw.
"""
from __future__ import annotations

import concurrent.futures as _futures
import os
from dataclasses import dataclass, replace

import numpy as np
import torch

DT_F32, DT_F16, DT_BF16 = 0, 1, 2
LAYOUT_SHARED, LAYOUT_SLOTTED = 0, 1
IDS_DISTINCT, IDS_MAY_REPEAT = 0, 1
DTYPE_SIZE = {DT_F32: 4, DT_F16: 2, DT_BF16: 2}
DTYPE_NAME = {DT_F32: "f32", DT_F16: "f16", DT_BF16: "bf16"}
_TORCH_DTYPE = {DT_F32: torch.float32, DT_F16: torch.float16, DT_BF16: torch.bfloat16}

# tensor tags for seeding
_T_WEIGHT, _T_X, _T_LOGITS, _T_BIAS, _T_IDS, _T_GATES = 1, 2, 3, 4, 5, 6


def _seed(*parts: int) -> int:
    state = np.random.SeedSequence([int(p) for p in parts]).generate_state(2, np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & ((1 << 62) - 1)


def generator(*parts: int) -> torch.Generator:
    return torch.Generator().manual_seed(_seed(*parts))


@dataclass(frozen=True)
class Workload:
    """One seeded synthetic problem: the full shape key plus how to draw it.

    ids_kind:   "logits"   -> ids come from routing N(0,1) logits + U(-0.1,0.1) bias
                "random"   -> top_k distinct experts per token, uniform
                "balanced" -> id = (t + s) mod E     (every expert equally loaded)
                "skewed"   -> id = s                 (experts 0..top_k-1 take every token)
                "repeat"   -> id = t mod E           (ids repeat inside a token)
    gates_kind: "routed"   -> gates from the router
                "softmax"  -> softmax of N(0,1) over the slots of each token
                "uniform"  -> 1/top_k
    """

    name: str
    dtype: int
    m: int
    n: int
    k: int
    top_k: int
    n_experts: int
    stride: int  # bytes between consecutive experts
    layout: int
    multiplicity: int
    seed: int
    w_std: float
    ids_kind: str
    gates_kind: str
    arith: int = 0  # eidm_arith: 0 the f32 order, 1 the split-16 matrix-core order

    @property
    def routed_rows(self) -> int:
        return self.m * self.top_k

    @property
    def input_rows(self) -> int:
        return self.routed_rows if self.layout == LAYOUT_SLOTTED else self.m

    @property
    def weight_bytes(self) -> int:
        return (self.n_experts - 1) * self.stride + self.n * self.k * DTYPE_SIZE[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _dense_stride(dtype: int, n: int, k: int) -> int:
    return n * k * DTYPE_SIZE[dtype]


WORKLOADS = {
    # plumbing: m=4, k=64, n=32, 8 experts, top-2, f32 weights N(0,0.1)
    "tiny": Workload("tiny", DT_F32, 4, 32, 64, 2, 8, _dense_stride(DT_F32, 32, 64),
                     LAYOUT_SHARED, IDS_DISTINCT, 1, 0.1, "random", "softmax"),
    # decode: one token, top-8 of 256 bf16 experts [1536, 4096]
    "decode": Workload("decode", DT_BF16, 1, 1536, 4096, 8, 256, _dense_stride(DT_BF16, 1536, 4096),
                       LAYOUT_SHARED, IDS_DISTINCT, 2, 0.02, "logits", "routed"),
    # prefill, every expert gets exactly 32 rows
    "prefill_balanced": Workload("prefill_balanced", DT_BF16, 512, 768, 2048, 8, 128,
                                 _dense_stride(DT_BF16, 768, 2048), LAYOUT_SHARED, IDS_DISTINCT,
                                 3, 0.02, "balanced", "uniform"),
    # prefill, experts 0..7 get all 512 tokens each
    "prefill_skewed": Workload("prefill_skewed", DT_BF16, 512, 768, 2048, 8, 128,
                               _dense_stride(DT_BF16, 768, 2048), LAYOUT_SHARED, IDS_DISTINCT,
                               3, 0.02, "skewed", "uniform"),
    # down projection with one input row per (token, slot)
    "down_proj": Workload("down_proj", DT_F16, 2048, 2048, 768, 8, 256, _dense_stride(DT_F16, 2048, 768),
                          LAYOUT_SLOTTED, IDS_DISTINCT, 5, 0.02, "logits", "routed"),
}


def small(name: str, **kw) -> Workload:
    """A small variant of a named workload with the same value recipe."""
    wl = WORKLOADS[name].with_(name=name + "_small", **kw)
    if "stride" not in kw:
        wl = wl.with_(stride=_dense_stride(wl.dtype, wl.n, wl.k))
    return wl


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def expert_weights(wl: Workload, e: int) -> torch.Tensor:
    """Expert e's [n, k] matrix in its native dtype (CPU)."""
    g = generator(wl.seed, _T_WEIGHT, e)
    w = torch.randn((wl.n, wl.k), generator=g, dtype=torch.float32)
    w.mul_(wl.w_std)
    return w.to(_TORCH_DTYPE[wl.dtype])


def expert_weights_f64(wl: Workload, e: int) -> np.ndarray:
    return expert_weights(wl, e).to(torch.float64).numpy()


def weight_bytes(wl: Workload) -> np.ndarray:
    """The whole weight buffer as bytes (expert e at byte e*stride; padding is 0)."""
    buf = np.zeros(wl.weight_bytes, dtype=np.uint8)
    body = wl.n * wl.k * DTYPE_SIZE[wl.dtype]
    for e in range(wl.n_experts):
        raw = expert_weights(wl, e).contiguous().view(torch.uint8).numpy().reshape(-1)
        buf[e * wl.stride: e * wl.stride + body] = raw
    return buf


def fill_weights(wl: Workload, dest: torch.Tensor, threads: int | None = None) -> None:
    """Write the weight buffer into `dest` (a uint8 tensor of >= weight_bytes,
    on any device), drawing experts in parallel on host threads."""
    assert dest.dtype == torch.uint8 and dest.numel() >= wl.weight_bytes
    body = wl.n * wl.k * DTYPE_SIZE[wl.dtype]
    if wl.stride != body:
        dest.zero_()
    threads = threads or min(16, os.cpu_count() or 4)

    def one(e: int) -> None:
        raw = expert_weights(wl, e).contiguous().view(torch.uint8).reshape(-1)
        dest[e * wl.stride: e * wl.stride + body].copy_(raw)

    with _futures.ThreadPoolExecutor(threads) as pool:
        list(pool.map(one, range(wl.n_experts)))


# --------------------------------------------------------------------------
# activations, router inputs, ids, gates
# --------------------------------------------------------------------------

def activations(wl: Workload) -> np.ndarray:
    """f32 [input_rows, k] ~ N(0, 1)."""
    g = generator(wl.seed, _T_X)
    return torch.randn((wl.input_rows, wl.k), generator=g, dtype=torch.float32).numpy()


def router_logits(wl: Workload) -> np.ndarray:
    """f32 [m, n_experts] ~ N(0, 1)."""
    g = generator(wl.seed, _T_LOGITS)
    return torch.randn((wl.m, wl.n_experts), generator=g, dtype=torch.float32).numpy()


def router_bias(wl: Workload) -> np.ndarray:
    """f32 [n_experts] ~ U(-0.1, 0.1): the per-expert selection bias."""
    g = generator(wl.seed, _T_BIAS)
    u = torch.rand((wl.n_experts,), generator=g, dtype=torch.float32)
    return (u * 0.2 - 0.1).numpy()


def profile_ids(m: int, top_k: int, n_experts: int, kind: str) -> np.ndarray:
    """Deterministic routing profiles (u32 [m, top_k])."""
    t = np.arange(m, dtype=np.int64)[:, None]
    s = np.arange(top_k, dtype=np.int64)[None, :]
    if kind == "balanced":
        ids = (t + s) % n_experts
    elif kind == "skewed":
        ids = np.broadcast_to(s, (m, top_k))
    elif kind == "repeat":
        ids = np.broadcast_to(t % n_experts, (m, top_k))
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(ids, dtype=np.uint32)


def random_distinct_ids(wl: Workload) -> np.ndarray:
    g = generator(wl.seed, _T_IDS)
    out = np.empty((wl.m, wl.top_k), dtype=np.uint32)
    for t in range(wl.m):
        out[t] = torch.randperm(wl.n_experts, generator=g)[: wl.top_k].numpy()
    return out


def ids(wl: Workload) -> np.ndarray:
    """ids for workloads that do not route from logits."""
    if wl.ids_kind == "random":
        return random_distinct_ids(wl)
    if wl.ids_kind in ("balanced", "skewed", "repeat"):
        return profile_ids(wl.m, wl.top_k, wl.n_experts, wl.ids_kind)
    raise ValueError(f"{wl.name}: ids come from the router")


def gates(wl: Workload) -> np.ndarray:
    """gates for workloads that do not route from logits (f32 [m, top_k])."""
    if wl.gates_kind == "uniform":
        return np.full((wl.m, wl.top_k), 1.0 / wl.top_k, dtype=np.float32)
    if wl.gates_kind == "softmax":
        g = generator(wl.seed, _T_GATES)
        z = torch.randn((wl.m, wl.top_k), generator=g, dtype=torch.float64)
        return torch.softmax(z, dim=1).to(torch.float32).numpy()
    raise ValueError(f"{wl.name}: gates come from the router")


def random_f32(shape, *seed_parts, std: float = 1.0) -> np.ndarray:
    g = generator(*seed_parts)
    return (torch.randn(tuple(shape), generator=g, dtype=torch.float32) * std).numpy()


# --------------------------------------------------------------------------
# the deterministic fills of the mlx-native dense_matmul_id_auto.rs tests
# --------------------------------------------------------------------------

_ADVERSARIAL = np.array([1.0009766, -1.0009766,
                         np.frombuffer(np.uint32(0x3F800001).tobytes(), np.float32)[0],
                         np.frombuffer(np.uint32(0xBF800001).tobytes(), np.float32)[0],
                         0.33333334, -0.14285715, 0.000012345679, -0.000009765625],
                        dtype=np.float32)


def adversarial_activations(rows: int, k: int) -> np.ndarray:
    """The calibration input pattern of fn calibration_buffers: eight bases
    (including 1 + 2^-23 and -(1 + 2^-23)) picked by index, scaled by
    1 + ((17 i) mod 11) / 4096 in f32."""
    i = np.arange(rows * k, dtype=np.int64)
    base = _ADVERSARIAL[(i * 5 + i // k) % 8]
    scale = (np.float32(1.0) + ((i * 17) % 11).astype(np.float32) / np.float32(4096.0)).astype(np.float32)
    return (base * scale).astype(np.float32).reshape(rows, k)


def modular_fill(count: int, seed: int, mul: int = 19, smul: int = 37, mod: int = 257,
                 off: int = 128, div: int = 263) -> np.ndarray:
    """((i*mul + seed*smul) mod mod - off) / div in f32: the weight fill of the
    page's injected-failure cases (19, 37, 257, 128, 263) and of its A-B-A
    case (17, 43, 251, 125, 257)."""
    i = np.arange(count, dtype=np.int64)
    return ((((i * mul + seed * smul) % mod).astype(np.float32) - np.float32(off)) / np.float32(div)).astype(np.float32)


# --------------------------------------------------------------------------
# the expert FFN: gate/up (shared layout) -> silu * up -> down (slotted)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class FfnWorkload:
    """A seeded mixture-of-experts FFN: per expert W_gate, W_up [inter, hidden]
    and W_down [hidden, inter] in one native dtype, N(0, w_std); tokens x
    [m, hidden] ~ N(0, 1); routed from N(0, 1) logits with a U(-0.1, 0.1)
    selection bias."""

    name: str
    dtype: int
    m: int
    hidden: int
    inter: int
    top_k: int
    n_experts: int
    seed: int
    w_std: float

    def part(self, which: str) -> Workload:
        """The matmul_id problem of one projection ("gate", "up", "down")."""
        size = DTYPE_SIZE[self.dtype]
        if which in ("gate", "up"):
            return Workload(f"{self.name}_{which}", self.dtype, self.m, self.inter, self.hidden, self.top_k,
                            self.n_experts, self.inter * self.hidden * size, LAYOUT_SHARED, IDS_DISTINCT,
                            self.seed * 10 + (1 if which == "gate" else 2), self.w_std, "logits", "routed")
        return Workload(f"{self.name}_down", self.dtype, self.m, self.hidden, self.inter, self.top_k,
                        self.n_experts, self.hidden * self.inter * size, LAYOUT_SLOTTED, IDS_DISTINCT,
                        self.seed * 10 + 3, self.w_std, "logits", "routed")

    def with_(self, **kw) -> "FfnWorkload":
        return replace(self, **kw)


FFN_WORKLOADS = {
    # the prefill FFN whose projections are the prefill shapes above:
    # gate/up [768, 2048] like the balanced config, down [2048, 768] like the down projection
    "ffn_prefill": FfnWorkload("ffn_prefill", DT_BF16, 512, 2048, 768, 8, 128, 7, 0.02),
}


def ffn_inputs(fw: FfnWorkload):
    """-> (x f32 [m, hidden], logits f32 [m, E], bias f32 [E])."""
    gate = fw.part("gate")
    return activations(gate), router_logits(gate), router_bias(gate)
