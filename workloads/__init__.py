"""Seeded synthetic inputs for the routed LoRA fold.

Shapes, value distributions and routing structure follow the workloads that the
routed-LoRA pages describe (decode BGMV on attention and FFN projections, MoE
decode gather-fold, MoE grouped prefill fold).  There is no public dataset for
this method; every array here is drawn from numpy's PCG64 with a fixed seed and
a fixed draw order.

This module holds none of the fold's arithmetic.  It draws random numbers and
builds index structures (slot ids, top-k expert choices, expert-sorted order).
BF16 values are made by drawing float32 and keeping the upper 16 bits
(truncation toward zero), so each value is exactly representable in BF16 and no
rounding rule of the method is involved.  Arrays of BF16 values are returned as
their uint16 bit patterns.

Both the CPU oracle and the GPU path consume these inputs; neither side's
results ever flow back into them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

SEED_BASE = 20261202


def rng_for(config_index: int, salt: int = 0) -> np.random.Generator:
    """Generator for a workload: seed = 20261202 + config index (+ salt)."""
    return np.random.Generator(np.random.PCG64(SEED_BASE + config_index + 1000 * salt))


def bf16_trunc(a) -> np.ndarray:
    """float32 values -> uint16 BF16 bit patterns by dropping the low 16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _normal(rng, shape, std=1.0):
    return bf16_trunc(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def _uniform(rng, shape, bound):
    return bf16_trunc(rng.uniform(-bound, bound, size=shape).astype(np.float32))


@dataclass
class Adapter:
    """One adapted module of one adapter, in PEFT layout (true rank, no padding).

    A is ``[rank, k_in]`` and B is ``[n_out, rank]`` (uint16 BF16 bits).
    ``expert`` is ``None`` for dense modules and the expert id for MoE experts.
    """

    slot: int
    rank: int
    alpha: float
    use_rslora: bool
    A: np.ndarray
    B: np.ndarray
    expert: Optional[int] = None


@dataclass
class BgmvCall:
    """One routed fold call: a module (route + pool) applied to a batch."""

    module: str
    k_in: int
    n_out: int
    max_rank: int
    max_loras: int
    adapters: List[Adapter]
    x_buf: str
    x_row_stride: int
    out_buf: str
    out_offset: int
    out_row_stride: int


@dataclass
class BgmvWorkload:
    name: str
    n: int
    seq_slot: np.ndarray  # int32 [n]
    buffers: Dict[str, np.ndarray]  # uint16 flat buffers (x inputs and fold outputs)
    calls: List[BgmvCall]


@dataclass
class MoeGatherWorkload:
    name: str
    num_tokens: int
    top_k: int
    num_experts: int
    k_in: int
    n_out: int
    max_rank: int
    max_loras: int
    indices: np.ndarray  # int32 [num_tokens*top_k], flat row rho = t*top_k + j
    row_adapter: Optional[np.ndarray]  # int32 [num_tokens] or None
    x: np.ndarray  # uint16 [n_rows, k_in]
    base: np.ndarray  # uint16 [n_rows, n_out]
    adapters: List[Adapter]

    @property
    def n_rows(self) -> int:
        return self.num_tokens * self.top_k


@dataclass
class GroupedProj:
    name: str
    k_in: int
    n_out: int
    x_gather: bool
    x: np.ndarray  # uint16 [te, k_in] sorted (x_gather=False) or [num_tokens, k_in]
    base: np.ndarray  # uint16 [te, n_out]
    adapters: List[Adapter]


@dataclass
class MoeGroupedWorkload:
    name: str
    num_tokens: int
    top_k: int
    num_experts: int
    te: int
    max_rank: int
    max_loras: int
    cap: int
    expert_offsets: np.ndarray  # int32 [num_experts+1]
    sorted_token_ids: np.ndarray  # int32 [te]
    row_adapter: Optional[np.ndarray]  # int32 [num_tokens] or None
    projections: List[GroupedProj]
    # ground truth kept from construction, for routing checks
    sorted_expert: np.ndarray = field(default=None)  # int32 [te]
    sorted_topk_pos: np.ndarray = field(default=None)  # int32 [te]


# ---------------------------------------------------------------------------
# adapters
# ---------------------------------------------------------------------------

def make_adapter(rng, slot, rank, k_in, n_out, alpha, use_rslora, expert=None):
    bound = 1.0 / np.sqrt(k_in)
    A = _uniform(rng, (rank, k_in), bound)
    B = _normal(rng, (n_out, rank), 0.02)
    return Adapter(slot=slot, rank=rank, alpha=float(alpha), use_rslora=bool(use_rslora),
                   A=A, B=B, expert=expert)


def _dense_adapters(rng, max_loras, ranks, k_in, n_out, alpha, rslora_even=False,
                    absent=()):
    out = []
    for s in range(max_loras):
        if s in absent:
            continue
        r = int(rng.choice(ranks))
        out.append(make_adapter(rng, s, r, k_in, n_out, alpha,
                                use_rslora=(rslora_even and s % 2 == 0)))
    return out


def _set_base_rows(rng, seq_slot, count):
    idx = rng.choice(len(seq_slot), size=count, replace=False)
    seq_slot[idx] = -1
    return seq_slot


# ---------------------------------------------------------------------------
# BGMV workloads
# ---------------------------------------------------------------------------

def bgmv_tiny(seed_index: int = 0) -> BgmvWorkload:
    """n=4, k_in=n_out=256, max_rank=8, two slots (true ranks 4 and 8), slots in {-1,0,1}."""
    rng = rng_for(seed_index)
    n, k_in, n_out, max_rank = 4, 256, 256, 8
    adapters = [make_adapter(rng, 0, 4, k_in, n_out, 16.0, False),
                make_adapter(rng, 1, 8, k_in, n_out, 16.0, False)]
    seq_slot = rng.integers(-1, 2, size=n).astype(np.int32)
    x = _normal(rng, (n, k_in))
    base = _normal(rng, (n, n_out))
    call = BgmvCall("proj", k_in, n_out, max_rank, 2, adapters, "x", k_in, "out", 0, n_out)
    return BgmvWorkload("tiny-bgmv n=4 k=256 r=8", n, seq_slot,
                        {"x": x.ravel(), "out": base.ravel()}, [call])


def bgmv_custom(seed_index, n, k_in, n_out, max_rank, max_loras, ranks, base_frac=0.1,
                x_row_stride=None, out_row_stride=None, out_offset=0, alpha=16.0,
                rslora_even=False, zipf=None, absent=()) -> BgmvWorkload:
    """A single-module routed batch with free shapes (used for parity sweeps)."""
    rng = rng_for(seed_index, salt=7)
    xs = x_row_stride or k_in
    os_ = out_row_stride or n_out
    adapters = _dense_adapters(rng, max_loras, ranks, k_in, n_out, alpha, rslora_even, absent)
    if zipf is not None:
        p = (np.arange(max_loras) + 1.0) ** (-zipf)
        p /= p.sum()
        seq_slot = rng.choice(max_loras, size=n, p=p).astype(np.int32)
    else:
        seq_slot = rng.integers(0, max_loras, size=n).astype(np.int32)
    _set_base_rows(rng, seq_slot, int(round(base_frac * n)))
    x = _normal(rng, (n, xs))
    base = _normal(rng, (n * os_ + out_offset,))
    call = BgmvCall("proj", k_in, n_out, max_rank, max_loras, adapters, "x", xs, "out",
                    out_offset, os_)
    return BgmvWorkload(f"bgmv n={n} k={k_in} nout={n_out} r={max_rank}", n, seq_slot,
                        {"x": x.ravel(), "out": base}, [call])


def bgmv_attn_decode(seed_index: int = 1, n: int = 64, hidden: int = 4096,
                     kv_out: int = 1024) -> BgmvWorkload:
    """Qwen3-8B-shaped attention side: q/k/v/o with k/v folded into [Q|K|V] rows.

    q: k_in=hidden -> n_out=hidden into a contiguous Q buffer; k, v: hidden -> kv_out
    into the interleaved qkv buffer (row stride hidden+2*kv_out, K at hidden, V at
    hidden+kv_out); o: hidden -> hidden on the attention output.  16 slots with true
    ranks from {8,16} (padded 16), alpha 16, 10% of rows on the base model.
    """
    rng = rng_for(seed_index)
    max_loras, max_rank = 16, 16
    qkv_stride = hidden + 2 * kv_out
    seq_slot = rng.integers(0, max_loras, size=n).astype(np.int32)
    _set_base_rows(rng, seq_slot, int(round(0.1 * n)))
    calls = []
    for module, n_out, xbuf, obuf, off, ostride in (
        ("q", hidden, "h", "q_out", 0, hidden),
        ("k", kv_out, "h", "qkv", hidden, qkv_stride),
        ("v", kv_out, "h", "qkv", hidden + kv_out, qkv_stride),
        ("o", hidden, "attn", "o_out", 0, hidden),
    ):
        ad = _dense_adapters(rng, max_loras, (8, 16), hidden, n_out, 16.0)
        calls.append(BgmvCall(module, hidden, n_out, max_rank, max_loras, ad, xbuf, hidden,
                              obuf, off, ostride))
    buffers = {
        "h": _normal(rng, (n, hidden)).ravel(),
        "attn": _normal(rng, (n, hidden)).ravel(),
        "q_out": _normal(rng, (n, hidden)).ravel(),
        "qkv": _normal(rng, (n, qkv_stride)).ravel(),
        "o_out": _normal(rng, (n, hidden)).ravel(),
    }
    return BgmvWorkload(f"attn-decode-bgmv n={n} hidden={hidden} q/k/v/o", n, seq_slot,
                        buffers, calls)


def bgmv_ffn_decode(seed_index: int = 2, n: int = 256, hidden: int = 4096,
                    inter: int = 12288) -> BgmvWorkload:
    """FFN side: gate/up hidden->inter, down inter->hidden; 32 slots, ranks {8,16,32,64}
    (padded 64), alpha 32 with rsLoRA scaling on even slots; slots Zipf(1.1) plus 5% base rows."""
    rng = rng_for(seed_index)
    max_loras, max_rank = 32, 64
    p = (np.arange(max_loras) + 1.0) ** (-1.1)
    p /= p.sum()
    seq_slot = rng.choice(max_loras, size=n, p=p).astype(np.int32)
    _set_base_rows(rng, seq_slot, int(round(0.05 * n)))
    calls = []
    for module, k_in, n_out, xbuf, obuf in (
        ("gate", hidden, inter, "h", "gate_out"),
        ("up", hidden, inter, "h", "up_out"),
        ("down", inter, hidden, "act", "down_out"),
    ):
        ad = _dense_adapters(rng, max_loras, (8, 16, 32, 64), k_in, n_out, 32.0,
                             rslora_even=True)
        calls.append(BgmvCall(module, k_in, n_out, max_rank, max_loras, ad, xbuf, k_in,
                              obuf, 0, n_out))
    buffers = {
        "h": _normal(rng, (n, hidden)).ravel(),
        "act": _normal(rng, (n, inter)).ravel(),
        "gate_out": _normal(rng, (n, inter)).ravel(),
        "up_out": _normal(rng, (n, inter)).ravel(),
        "down_out": _normal(rng, (n, hidden)).ravel(),
    }
    return BgmvWorkload(f"ffn-decode-bgmv n={n} {hidden}->{inter}->{hidden}", n, seq_slot,
                        buffers, calls)


def decode_routing(seed_index: int = 6, n: int = 64, max_loras: int = 16,
                   base_frac: float = 0.1) -> np.ndarray:
    """seq_slot of one decode batch shared by every layer of a step: slots
    uniform over 0..max_loras-1, base_frac of the rows on the base model."""
    rng = rng_for(seed_index)
    seq_slot = rng.integers(0, max_loras, size=n).astype(np.int32)
    return _set_base_rows(rng, seq_slot, int(round(base_frac * n)))


def decode_layer(layer: int, seq_slot: np.ndarray, seed_index: int = 6, hidden: int = 4096,
                 kv_out: int = 1024, inter: int = 12288, max_loras: int = 16,
                 ranks=(8, 16), alpha: float = 16.0) -> BgmvWorkload:
    """One decoder layer of Qwen3-8B shapes with every projection adapted: q
    hidden->hidden, k and v hidden->kv_out folded into [Q|K|V] rows (stride
    hidden+2*kv_out, K at hidden, V at hidden+kv_out), o hidden->hidden, gate and
    up hidden->inter, down inter->hidden.  The layer's own pools (max_loras
    slots, true ranks from `ranks`, padded to the largest) and activations are
    drawn from a generator seeded by the layer index; the batch's routing
    seq_slot is shared by every layer."""
    rng = rng_for(seed_index, salt=layer + 1)
    n = len(seq_slot)
    max_rank = max(ranks)
    qkv_stride = hidden + 2 * kv_out
    calls = []
    for module, k_in, n_out, xbuf, obuf, off, ostride in (
        ("q", hidden, hidden, "h", "q_out", 0, hidden),
        ("k", hidden, kv_out, "h", "qkv", hidden, qkv_stride),
        ("v", hidden, kv_out, "h", "qkv", hidden + kv_out, qkv_stride),
        ("o", hidden, hidden, "attn", "o_out", 0, hidden),
        ("gate", hidden, inter, "h2", "gate_out", 0, inter),
        ("up", hidden, inter, "h2", "up_out", 0, inter),
        ("down", inter, hidden, "act", "down_out", 0, hidden),
    ):
        ad = _dense_adapters(rng, max_loras, ranks, k_in, n_out, alpha)
        calls.append(BgmvCall(module, k_in, n_out, max_rank, max_loras, ad, xbuf, k_in, obuf,
                              off, ostride))
    buffers = {
        "h": _normal(rng, (n, hidden)).ravel(),
        "attn": _normal(rng, (n, hidden)).ravel(),
        "h2": _normal(rng, (n, hidden)).ravel(),
        "act": _normal(rng, (n, inter)).ravel(),
        "q_out": _normal(rng, (n, hidden)).ravel(),
        "qkv": _normal(rng, (n, qkv_stride)).ravel(),
        "o_out": _normal(rng, (n, hidden)).ravel(),
        "gate_out": _normal(rng, (n, inter)).ravel(),
        "up_out": _normal(rng, (n, inter)).ravel(),
        "down_out": _normal(rng, (n, hidden)).ravel(),
    }
    return BgmvWorkload(f"decode layer {layer} n={n} q/k/v/o/gate/up/down", n, seq_slot,
                        buffers, calls)


def lora_prefill(seed_index: int = 5, m: int = 4096, hidden: int = 4096, inter: int = 12288,
                 rank: int = 64, alpha: float = 32.0) -> BgmvWorkload:
    """Unrouted single adapter over a prefill batch (the apply_lora_delta path):
    m tokens through the FFN of Qwen3-8B shapes, gate/up hidden->inter and down
    inter->hidden, one adapter of rank 64 (scale alpha/r) on slot 0.  Every row
    uses the adapter (seq_slot is all zero, for the routed comparison)."""
    rng = rng_for(seed_index)
    calls = []
    for module, k_in, n_out, xbuf, obuf in (
        ("gate", hidden, inter, "h", "gate_out"),
        ("up", hidden, inter, "h", "up_out"),
        ("down", inter, hidden, "act", "down_out"),
    ):
        ad = [make_adapter(rng, 0, rank, k_in, n_out, alpha, False)]
        calls.append(BgmvCall(module, k_in, n_out, rank, 1, ad, xbuf, k_in, obuf, 0, n_out))
    buffers = {
        "h": _normal(rng, (m, hidden)).ravel(),
        "act": _normal(rng, (m, inter)).ravel(),
        "gate_out": _normal(rng, (m, inter)).ravel(),
        "up_out": _normal(rng, (m, inter)).ravel(),
        "down_out": _normal(rng, (m, hidden)).ravel(),
    }
    return BgmvWorkload(f"unrouted prefill m={m} {hidden}->{inter}->{hidden} r{rank}", m,
                        np.zeros(m, np.int32), buffers, calls)


# ---------------------------------------------------------------------------
# MoE workloads
# ---------------------------------------------------------------------------

def _expert_adapters(rng, max_loras, num_experts, n_adapted, ranks, k_in, n_out, alpha):
    out = []
    for s in range(max_loras):
        experts = np.sort(rng.choice(num_experts, size=n_adapted, replace=False))
        for e in experts:
            r = int(rng.choice(ranks))
            out.append(make_adapter(rng, s, r, k_in, n_out, alpha, False, expert=int(e)))
    return out


def moe_gather(seed_index: int = 3, num_tokens: int = 32, top_k: int = 8,
               num_experts: int = 128, k_in: int = 768, n_out: int = 2048,
               max_loras: int = 8, n_adapted: int = 64, ranks=(8, 16), max_rank: int = 16,
               with_row_adapter: bool = True) -> MoeGatherWorkload:
    """Decode down_proj gather-fold: each token's top_k experts distinct and uniform;
    flat slot-major rows rho = t*top_k + j; per adapter slot an independent subset of
    n_adapted experts carries an adapter; row_adapter[t] uniform in {-1, 0..max_loras-1}."""
    rng = rng_for(seed_index)
    indices = np.stack([rng.choice(num_experts, size=top_k, replace=False)
                        for _ in range(num_tokens)]).astype(np.int32).ravel()
    row_adapter = rng.integers(-1, max_loras, size=num_tokens).astype(np.int32)
    adapters = _expert_adapters(rng, max_loras, num_experts, n_adapted, ranks, k_in, n_out,
                                16.0)
    n_rows = num_tokens * top_k
    x = _normal(rng, (n_rows, k_in))
    base = _normal(rng, (n_rows, n_out))
    return MoeGatherWorkload(
        f"moe-gather tokens={num_tokens} top{top_k} E={num_experts} {k_in}->{n_out}",
        num_tokens, top_k, num_experts, k_in, n_out, max_rank, max_loras, indices,
        row_adapter if with_row_adapter else None, x, base, adapters)


def route_topk(rng, num_tokens, num_experts, top_k):
    """Router logits ~N(0,1) -> top_k experts per token (softmax is monotone, so the
    top_k of the logits); ties go to the lower expert id."""
    logits = rng.standard_normal(size=(num_tokens, num_experts), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :top_k].astype(np.int32)


def expert_sort(topk: np.ndarray, num_experts: int):
    """Expert-sorted layout of the (token, k) pairs: by expert, then token, then k.

    Returns (expert_offsets [E+1], sorted_token_ids [te], sorted_expert [te],
    sorted_topk_pos [te]).
    """
    num_tokens, top_k = topk.shape
    tok = np.repeat(np.arange(num_tokens, dtype=np.int64), top_k)
    pos = np.tile(np.arange(top_k, dtype=np.int64), num_tokens)
    exp = topk.ravel().astype(np.int64)
    order = np.lexsort((pos, tok, exp))
    counts = np.bincount(exp, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return (offsets, tok[order].astype(np.int32), exp[order].astype(np.int32),
            pos[order].astype(np.int32))


def moe_grouped(seed_index: int = 4, num_tokens: int = 4096, top_k: int = 8,
                num_experts: int = 128, hidden: int = 2048, inter: int = 768,
                max_loras: int = 4, n_adapted: int = 96, ranks=(16, 32), max_rank: int = 32,
                cap: int = 8192, projections=("down", "gate", "up"),
                with_row_adapter: bool = True) -> MoeGroupedWorkload:
    """Prefill grouped fold: router top_k over N(0,1) logits, expert-sorted rows.

    down: x = sorted post-SiLU activations [te, inter] -> n_out = hidden.
    gate/up: x = token-major input [num_tokens, hidden] gathered through
    sorted_token_ids -> n_out = inter.  Per adapter slot an independent subset of
    n_adapted experts is adapted; row_adapter[t] uniform in {-1, 0..max_loras-1}.
    """
    rng = rng_for(seed_index)
    topk = route_topk(rng, num_tokens, num_experts, top_k)
    offsets, stid, sexp, spos = expert_sort(topk, num_experts)
    te = num_tokens * top_k
    row_adapter = rng.integers(-1, max_loras, size=num_tokens).astype(np.int32)
    projs = []
    x_tok = None
    for name in projections:
        if name == "down":
            k_in, n_out, gather = inter, hidden, False
        else:
            k_in, n_out, gather = hidden, inter, True
        ad = _expert_adapters(rng, max_loras, num_experts, n_adapted, ranks, k_in, n_out,
                              16.0)
        if gather:
            if x_tok is None:
                x_tok = _normal(rng, (num_tokens, hidden))
            x = x_tok
        else:
            x = _normal(rng, (te, k_in))
        base = _normal(rng, (te, n_out))
        projs.append(GroupedProj(name, k_in, n_out, gather, x, base, ad))
    return MoeGroupedWorkload(
        f"moe-grouped tokens={num_tokens} top{top_k} E={num_experts} te={te} cap={cap}",
        num_tokens, top_k, num_experts, te, max_rank, max_loras, cap, offsets, stid,
        row_adapter if with_row_adapter else None, projs, sexp, spos)
