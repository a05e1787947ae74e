"""CPU oracle of the routed LoRA delta.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The library (``routed_lora_delta_amd``)
never imports, links or calls it, and this module imports nothing from the
library.  The two share no code; only the seeded input generators
(``workloads``) feed both.

What it computes, and where the pages say so:

* "Function apply_lora_bgmv" (rustdoc, description and STRIDES paragraphs):
  for every row i of a batch, s = seq_slot[i]; a negative slot, or a slot whose
  A/B table entry is 0, adds nothing.  Otherwise
  ``xa = bf16(x_i @ A_s^T)``, ``delta = bf16(xa @ B_s^T)`` and
  ``out_i = bf16(f32(out_i) + scale_s * f32(delta))``, the scale applied in
  fp32 after the delta has been rounded to BF16.  Both contractions run at the
  pool's padded max_rank.  Row strides are in elements.
* "Module lora_delta" (LoraPair, LoraRoute) and the lora_delta.rs listing
  (LoraPair, apply_lora_bgmv doc comment): A is ``[max_rank, k_in]``, B is
  ``[n_out, max_rank]``, both row-major BF16 with zero rows/columns past the
  adapter's rank; scale = alpha/r, or alpha/sqrt(r) with use_rslora, kept out
  of B.
* "Module lora_delta" and the lora_delta.rs listing (apply_lora_delta doc
  comment): the unrouted single-adapter delta, base_out[m, n_out] +=
  scale * (x @ a^T) @ b^T for one LoraPair, with the same rounding points as
  the routed fold (the pages state that the routed path is byte-identical to
  row-by-row calls of this one).
* "Module moe_lora_grouped" (moe_lora_grouped_down, moe_lora_gather_bgmv,
  pack_expert_tables, grouped_down_wc, grouped_down_windows,
  gather_row_token): the same fold for MoE experts, over expert-sorted rows of
  one chunk window (expert from the expert_offsets prefix sum, token from
  sorted_token_ids, optional x gather, xa at the window-local row) or over
  unsorted flat (token, top-k) rows (expert from indices[row], adapter from
  row_adapter[row / top_k]).

Precision.  The pages fix the BF16 rounding of xa and delta and an fp32 fold;
they do not state how the contractions accumulate.  Here each contraction is
the dot product of BF16 values computed in float64 (exact to far below BF16
resolution for these sizes) and rounded once, round-to-nearest-even, to BF16.
The fold is done in float32: the product scale*delta is rounded to float32,
then the sum with the base value is rounded to float32, then that is rounded
to BF16.

Readings where the pages are silent (each also listed with the design notes):
  * a slot is active iff 0 <= s < max_loras and both its A and B entries are
    present; s >= max_loras is treated as base-only;
  * xa rows of rows that do not fold are written as zeros;
  * MoE adapter identity: tables are [max_loras][num_experts]; row_adapter
    (or, when absent, slot 0) picks the row of the table;
  * grouped path: the adapter lookup uses t = sorted_token_ids[r] in both the
    gather and the non-gather mode; rows outside every expert span, experts
    beyond the table, unadapted pairs and, whenever sorted_token_ids is given,
    tokens outside [0, num_tokens) are skipped.

Pins (``tests/test_oracle.py``): BF16 rounding against hand-derived bit
patterns, exhaustive round trips and torch's float32->bfloat16 conversion;
scale closed forms; exact-rational brute force on tiny inputs; the textbook
single-adapter LoRA on integer-exact inputs (orientation and scale); pad
invariance; untouched base rows and strided regions; batched == per-row; the
fold's multiply-then-add order on a hand-derived case; closed-form routing
probes for the gather and grouped paths; full window == union of chunk
windows; the pure helpers against the statements on the moe_lora_grouped page.
Parity unpinned: the order in which a GPU sums a contraction (no page fixes
it), which the GPU tolerance absorbs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# BF16 <-> float, from the IEEE-754 binary formats
# ---------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite bfloat16


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns -> float64 (a BF16 value is the upper half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_bf16(v) -> np.ndarray:
    """Round real values (float64 or float32 arrays) to BF16, ties to even.

    BF16 keeps 8 significant bits.  In the binade [2^e, 2^(e+1)) the spacing is
    2^(e-7); below the normal range (e < -126) the spacing stays 2^-133
    (subnormals are kept).  A value is divided by the spacing (exact: a power
    of two), rounded to an integer with ties to even, and scaled back.  Results
    above the largest finite BF16 become infinity; NaN becomes the quiet NaN
    with the sign kept; the sign of zero is kept.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    a_fin = np.where(finite, a, 0.0)
    _, E = np.frexp(a_fin)  # a = m * 2^E with m in [0.5, 1)
    e = np.maximum(E - 1, -126)
    q = np.ldexp(1.0, e - 7)
    r = np.rint(a_fin / q) * q
    r = np.where(r > BF16_MAX, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    mag = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mag = np.where(np.isnan(v), np.uint16(0x7FC0), mag)
    sign = np.signbit(v).astype(np.uint16) << np.uint16(15)
    return (mag | sign).astype(np.uint16)


# ---------------------------------------------------------------------------
# adapter pack (install time)
# ---------------------------------------------------------------------------

def f16_to_bf16(bits) -> np.ndarray:
    """Adapter install ("Module lora_delta": PEFT tensors converted F16 -> BF16 on
    the host): the F16 value (numpy's float16 decoding, exact in float64)
    rounded to BF16 by round_bf16."""
    return round_bf16(np.asarray(bits, np.uint16).view(np.float16).astype(np.float64))


def scale_for(alpha: float, rank: int, use_rslora: bool) -> np.float32:
    """LoraPair scale: lora_alpha / r, or lora_alpha / sqrt(r) under use_rslora
    (lora_delta.rs listing, LoraPair doc comment).  Computed in double and
    rounded once to float32."""
    if rank <= 0:
        raise ValueError("rank must be positive")
    d = alpha / math.sqrt(rank) if use_rslora else alpha / rank
    return np.float32(d)


@dataclass
class SlotWeights:
    """A packed (padded) adapter module: A [max_rank, k_in], B [n_out, max_rank]
    as BF16 bits, and the fp32 scale.  A or B may be None (table entry 0)."""

    A: Optional[np.ndarray]
    B: Optional[np.ndarray]
    scale: np.float32
    _a64: Optional[np.ndarray] = None
    _b64: Optional[np.ndarray] = None

    @property
    def active(self) -> bool:
        return self.A is not None and self.B is not None

    def a64(self):
        if self._a64 is None:
            self._a64 = bf16_to_f64(self.A)
        return self._a64

    def b64(self):
        if self._b64 is None:
            self._b64 = bf16_to_f64(self.B)
        return self._b64


def pad_adapter(A: np.ndarray, B: np.ndarray, max_rank: int) -> Tuple[np.ndarray, np.ndarray]:
    """Pool layout of one PEFT pair: A [rank, k_in] -> [max_rank, k_in] with zero
    rows after rank; B [n_out, rank] -> [n_out, max_rank] with zero columns after
    rank (the pool is zeroed before packing: lora_delta.rs header invariants)."""
    rank, k_in = A.shape
    n_out = B.shape[0]
    if B.shape[1] != rank or rank > max_rank:
        raise ValueError("bad adapter shapes")
    Ap = np.zeros((max_rank, k_in), np.uint16)
    Ap[:rank] = A
    Bp = np.zeros((n_out, max_rank), np.uint16)
    Bp[:, :rank] = B
    return Ap, Bp


def pack_slots(adapters: Sequence, max_loras: int, max_rank: int) -> List[Optional[SlotWeights]]:
    """Slot-keyed route of one module: entry s holds slot s's padded pair and
    scale, None where the slot does not adapt the module (table entry 0).  A
    repeated slot keeps the last entry."""
    slots: List[Optional[SlotWeights]] = [None] * max_loras
    for ad in adapters:
        if not (0 <= ad.slot < max_loras):
            raise ValueError("slot out of range")
        Ap, Bp = pad_adapter(ad.A, ad.B, max_rank)
        slots[ad.slot] = SlotWeights(Ap, Bp, scale_for(ad.alpha, ad.rank, ad.use_rslora))
    return slots


def pack_expert_pairs(adapters: Sequence, max_loras: int, num_experts: int,
                      max_rank: int) -> List[List[Optional[SlotWeights]]]:
    """MoE route: [max_loras][num_experts] table of padded pairs (None = unadapted)."""
    pairs = [[None] * num_experts for _ in range(max_loras)]
    for ad in adapters:
        Ap, Bp = pad_adapter(ad.A, ad.B, max_rank)
        pairs[ad.slot][ad.expert] = SlotWeights(Ap, Bp, scale_for(ad.alpha, ad.rank,
                                                                  ad.use_rslora))
    return pairs


# ---------------------------------------------------------------------------
# pure helpers ("Module moe_lora_grouped", Functions and Constants)
# ---------------------------------------------------------------------------

M_TILE = 64  # MLG_M_TILE


def pack_expert_tables(entries):
    """(expert_id, a_addr, b_addr, scale) entries -> dense tables indexed by expert.

    n_experts = max expert id + 1; 0 / 0.0 at every unadapted expert; None for
    no entries; a repeated expert id keeps the last entry."""
    if len(entries) == 0:
        return None
    n = max(int(e[0]) for e in entries) + 1
    a = [0] * n
    b = [0] * n
    sc = [np.float32(0.0)] * n
    for eid, aa, bb, s in entries:
        a[eid], b[eid], sc[eid] = int(aa), int(bb), np.float32(s)
    return n, a, b, sc


def grouped_down_windows(total_rows: int, cap: int) -> List[Tuple[int, int]]:
    """Contiguous [start, end) windows of at most cap rows covering 0..total_rows."""
    if cap <= 0:
        raise ValueError("cap must be positive")
    out = []
    start = 0
    while start < total_rows:
        end = min(start + cap, total_rows)
        out.append((start, end))
        start = end
    return out


def grouped_down_wc(row_offset: int, row_end: int) -> int:
    """m-tile count of one window: ceil((row_end-row_offset)/64), at least 1."""
    return max(1, -(-(row_end - row_offset) // M_TILE))


def gather_row_token(row: int, top_k: int) -> int:
    """Owning token of a flat (token, top-k position) row."""
    return row // top_k


# ---------------------------------------------------------------------------
# the fold
# ---------------------------------------------------------------------------

def fold_row(x_row_bits: np.ndarray, w: SlotWeights, out_row_bits: np.ndarray):
    """One row: xa = bf16(x @ A^T); delta = bf16(xa @ B^T);
    out = bf16(f32(out) + f32(scale * f32(delta)))."""
    xa = round_bf16(w.a64() @ bf16_to_f64(x_row_bits))
    d = round_bf16(w.b64() @ bf16_to_f64(xa))
    t = np.float32(w.scale) * bf16_to_f32(d)  # float32 product, rounded once
    s = bf16_to_f32(out_row_bits) + t  # float32 sum, rounded once
    return xa, round_bf16(s)


def bgmv(slots: List[Optional[SlotWeights]], k_in: int, n_out: int, max_rank: int,
         x: np.ndarray, x_row_stride: int, seq_slot: np.ndarray, n: int,
         base_out: np.ndarray, out_offset: int, out_row_stride: int):
    """Routed BGMV over n rows.  x and base_out are flat BF16 buffers; row i of x
    starts at i*x_row_stride, row i of the output region at
    out_offset + i*out_row_stride and spans n_out elements.

    Returns (xa [n, max_rank] BF16 bits, folded copy of base_out)."""
    xa = np.zeros((n, max_rank), np.uint16)
    out = np.array(base_out, dtype=np.uint16, copy=True)
    for i in range(n):
        s = int(seq_slot[i])
        if s < 0 or s >= len(slots) or slots[s] is None or not slots[s].active:
            continue
        xrow = x[i * x_row_stride: i * x_row_stride + k_in]
        o0 = out_offset + i * out_row_stride
        xa[i], out[o0: o0 + n_out] = fold_row(xrow, slots[s], out[o0: o0 + n_out])
    return xa, out


def lora_delta(w: SlotWeights, k_in: int, n_out: int, max_rank: int, x: np.ndarray,
               x_row_stride: int, m: int, base_out: np.ndarray, out_offset: int,
               out_row_stride: int):
    """Unrouted delta of one adapter pair over m rows (apply_lora_delta), written
    as matrices: XA = bf16(X @ A^T) [m, max_rank], D = bf16(XA @ B^T) [m, n_out],
    OUT = bf16(f32(OUT) + f32(scale * f32(D))).  Row i of x starts at
    i*x_row_stride, row i of the output region at out_offset + i*out_row_stride.
    Returns (xa [m, max_rank] BF16 bits, folded copy of base_out)."""
    out = np.array(base_out, dtype=np.uint16, copy=True)
    if m == 0:
        return np.zeros((0, max_rank), np.uint16), out
    rows_x = np.arange(m)[:, None] * x_row_stride + np.arange(k_in)[None, :]
    X = bf16_to_f64(np.asarray(x)[rows_x])                       # [m, k_in]
    XA = round_bf16(X @ w.a64().T)                                # [m, max_rank]
    D = round_bf16(bf16_to_f64(XA) @ w.b64().T)                   # [m, n_out]
    rows_o = out_offset + np.arange(m)[:, None] * out_row_stride + np.arange(n_out)[None, :]
    T = np.float32(w.scale) * bf16_to_f32(D)                      # float32 products
    S = bf16_to_f32(out[rows_o]) + T                              # float32 sums
    out[rows_o] = round_bf16(S)
    return XA, out


def moe_gather(pairs, num_experts: int, k_in: int, n_out: int, max_rank: int,
               x: np.ndarray, x_row_stride: int, indices: np.ndarray,
               row_adapter: Optional[np.ndarray], top_k: int, n_rows: int,
               base_out: np.ndarray, out_row_stride: int):
    """Decode gather-fold over unsorted flat rows rho: expert e = indices[rho],
    token t = rho // top_k, slot s = row_adapter[t] (slot 0 when row_adapter is
    None).  Returns (xa [n_rows, max_rank], folded copy of base_out)."""
    max_loras = len(pairs)
    xa = np.zeros((n_rows, max_rank), np.uint16)
    out = np.array(base_out, dtype=np.uint16, copy=True)
    for rho in range(n_rows):
        t = gather_row_token(rho, top_k)
        s = int(row_adapter[t]) if row_adapter is not None else 0
        e = int(indices[rho])
        if not (0 <= s < max_loras and 0 <= e < num_experts):
            continue
        w = pairs[s][e]
        if w is None or not w.active:
            continue
        xrow = x[rho * x_row_stride: rho * x_row_stride + k_in]
        o0 = rho * out_row_stride
        xa[rho], out[o0: o0 + n_out] = fold_row(xrow, w, out[o0: o0 + n_out])
    return xa, out


def expert_owner(expert_offsets: np.ndarray, row_offset: int, row_end: int) -> np.ndarray:
    """For each row of [row_offset, row_end): the expert e with
    off[e] <= r < off[e+1], or -1 when no span holds the row.  The offsets are a
    prefix sum, so they must not decrease."""
    off = np.asarray(expert_offsets, dtype=np.int64)
    if np.any(np.diff(off) < 0):
        raise ValueError("expert_offsets must be non-decreasing")
    owner = np.full(row_end - row_offset, -1, np.int64)
    for e in range(len(off) - 1):
        lo = max(int(off[e]), row_offset)
        hi = min(int(off[e + 1]), row_end)
        if lo < hi:
            owner[lo - row_offset: hi - row_offset] = e
    return owner


def moe_grouped(pairs, num_experts: int, k_in: int, n_out: int, max_rank: int,
                x: np.ndarray, x_row_stride: int, x_gather: bool, num_tokens: int,
                expert_offsets: np.ndarray, sorted_token_ids: Optional[np.ndarray],
                row_adapter: Optional[np.ndarray], row_offset: int, row_end: int,
                base_out: np.ndarray, out_row_stride: int):
    """Grouped fold of one chunk window [row_offset, row_end) of expert-sorted rows.

    Row r: expert e from the expert_offsets spans (an offsets array may list
    more experts than the table holds: a row of an expert past the table is
    skipped); t = sorted_token_ids[r], read whenever the map is given, and a
    token outside [0, num_tokens) skips the row (the map may be None only
    when neither the x gather nor row_adapter needs it); slot
    s = row_adapter[t] (slot 0 when row_adapter is None); the x row is x[t]
    when x_gather else x[r]; base_out row r is folded in place; xa is written
    at the window-local row r - row_offset.
    Returns (xa [row_end-row_offset, max_rank], folded copy of base_out)."""
    max_loras = len(pairs)
    nloc = row_end - row_offset
    xa = np.zeros((max(nloc, 0), max_rank), np.uint16)
    out = np.array(base_out, dtype=np.uint16, copy=True)
    if nloc <= 0:
        return xa, out
    owner = expert_owner(expert_offsets, row_offset, row_end)
    if (x_gather or row_adapter is not None) and sorted_token_ids is None:
        raise ValueError("sorted_token_ids is needed for the x gather and row_adapter")
    need_token = sorted_token_ids is not None
    for r in range(row_offset, row_end):
        e = int(owner[r - row_offset])
        if e < 0 or e >= num_experts:
            continue
        t = int(sorted_token_ids[r]) if need_token else -1
        if need_token and not (0 <= t < num_tokens):
            continue
        s = int(row_adapter[t]) if row_adapter is not None else 0
        if not (0 <= s < max_loras):
            continue
        w = pairs[s][e]
        if w is None or not w.active:
            continue
        xr = t if x_gather else r
        xrow = x[xr * x_row_stride: xr * x_row_stride + k_in]
        o0 = r * out_row_stride
        xa[r - row_offset], out[o0: o0 + n_out] = fold_row(xrow, w, out[o0: o0 + n_out])
    return xa, out
