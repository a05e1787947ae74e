"""The bench's algorithmic byte counts, checked on the CPU against a count that
walks the rows one by one (the roofline's `achieved` divides these bytes by a
measured launch time, so a miscount would misstate every fraction of peak).

Per call the count is: the x rows that fold (for a gathered x, the distinct
tokens), A and B of every distinct (slot[, expert]) pair the call touches, the
base rows read and written, xa written and read, and the index arrays.  For the
MoE gate+up pair launch and the BGMV one-pass form the read-once figure takes
x once over the union of the rows (tokens) any of the launch's calls folds, and
no xa read-back."""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench as B  # noqa: E402
import workloads as W  # noqa: E402


def _walk_bgmv(wl, c):
    have = {a.slot for a in c.adapters}
    x_rows, slots = 0, set()
    for i in range(wl.n):
        s = int(wl.seq_slot[i])
        if s in have:
            x_rows += 1
            slots.add(s)
    R = c.max_rank
    shrink = 2 * x_rows * c.k_in + 2 * len(slots) * R * c.k_in + 2 * wl.n * R + 4 * wl.n
    expand = (2 * len(slots) * c.n_out * R + 2 * x_rows * R + 4 * x_rows * c.n_out
              + 4 * wl.n)
    return shrink, expand


def test_bgmv_bytes_match_a_row_walk():
    for wl in (W.bgmv_tiny(), W.bgmv_custom(7, 40, 256, 136, 16, 5, (8, 16), base_frac=0.3)):
        for c in wl.calls:
            sb, eb, fl, n_act = B.bgmv_bytes(wl, c)
            assert (sb, eb) == _walk_bgmv(wl, c)
            assert n_act == sum(int(s) in {a.slot for a in c.adapters} for s in wl.seq_slot)
            assert fl == 2 * n_act * c.max_rank * (c.k_in + c.n_out)


def _small_grouped():
    return W.moe_grouped(seed_index=11, num_tokens=96, top_k=4, num_experts=16, hidden=256,
                         inter=128, max_loras=3, n_adapted=10, ranks=(8, 16), max_rank=16,
                         cap=128)


def _walk_grouped(wl, p, lo, hi):
    """(distinct x tokens or rows, distinct pairs, folding rows) of window [lo, hi)."""
    pairs = {(a.slot, a.expert) for a in p.adapters}
    toks, seen, n_act = set(), set(), 0
    for r in range(lo, hi):
        t = int(wl.sorted_token_ids[r])
        s = int(wl.row_adapter[t])
        e = int(np.searchsorted(wl.expert_offsets, r, side="right") - 1)
        if (s, e) in pairs:
            n_act += 1
            toks.add(t)
            seen.add((s, e))
    return toks, seen, n_act


def test_grouped_window_bytes_match_a_row_walk():
    wl = _small_grouped()
    R = wl.max_rank
    for p in wl.projections:
        for lo in range(0, wl.te, wl.cap):
            hi = min(lo + wl.cap, wl.te)
            toks, seen, n_act = _walk_grouped(wl, p, lo, hi)
            x_rows = len(toks) if p.x_gather else n_act
            idx = 4 * (2 * (hi - lo) + wl.num_experts + 1)
            sb, eb, _, na = B.grouped_window_bytes(wl, p, lo, hi)
            assert na == n_act
            assert sb == 2 * (x_rows * p.k_in + len(seen) * R * p.k_in + (hi - lo) * R) + idx
            assert eb == 2 * (len(seen) * p.n_out * R + n_act * R + 2 * n_act * p.n_out) + idx


def test_pair_read_once_bytes_take_x_once_and_no_xa_read():
    wl = _small_grouped()
    P = {p.name: p for p in wl.projections}
    g, u = P["gate"], P["up"]
    R = wl.max_rank
    for lo in range(0, wl.te, wl.cap):
        hi = min(lo + wl.cap, wl.te)
        tg, _, ng = _walk_grouped(wl, g, lo, hi)
        tu, _, nu = _walk_grouped(wl, u, lo, hi)
        sb, eb, _, _ = B.grouped_window_bytes(wl, g, lo, hi)
        sb2, eb2, _, _ = B.grouped_window_bytes(wl, u, lo, hi)
        got = B.grouped_pair_read_once_bytes(wl, g, u, lo, hi)
        # the calls' sum counts x of gate's tokens and of up's tokens, and xa
        # read back by both expands; the launch reads x of their union once
        want = (sb + eb + sb2 + eb2 - 2 * g.k_in * (len(tg) + len(tu) - len(tg | tu))
                - 2 * R * (ng + nu))
        assert got == want
        # a projection paired with itself reads its x once
        sp, ep, _, n = B.grouped_window_bytes(wl, g, lo, hi)
        assert B.grouped_pair_read_once_bytes(wl, g, g, lo, hi) == (
            2 * (sp + ep) - 2 * g.k_in * len(tg) - 4 * R * n)


def test_read_once_fields():
    assert B._read_once_fields([], 1e-5) == {}
    assert B._read_once_fields([100, None], 1e-5) == {}
    f = B._read_once_fields([8e6, 8e6], 1e-5)  # 8 MB in 10 us: 800 GB/s
    assert f["read_once_bytes_per_launch"] == 8000000
    assert abs(f["read_once_achieved"] - 800.0) < 1e-6
    assert abs(f["read_once_frac"] - 0.1) < 1e-9


def test_bgmv_read_once_bytes_take_x_once():
    wl = W.bgmv_attn_decode()
    qkv = [c for c in wl.calls if c.module in ("q", "k", "v")]
    total = sum(sum(B.bgmv_bytes(wl, c)[:2]) for c in qkv)
    rows = [r for r in range(wl.n)
            if any(int(wl.seq_slot[r]) in {a.slot for a in c.adapters} for c in qkv)]
    n_acts = [B.bgmv_bytes(wl, c)[3] for c in qkv]
    k_in, R = qkv[0].k_in, qkv[0].max_rank
    x_dup = 2 * k_in * (sum(n_acts) - len(rows))
    assert B.bgmv_read_once_bytes(wl, qkv, False) == total - x_dup
    assert B.bgmv_read_once_bytes(wl, qkv, True) == total - x_dup - 2 * R * sum(n_acts)
    # one call: only the xa read-back differs
    c = qkv[0]
    sb, eb, _, n_act = B.bgmv_bytes(wl, c)
    assert B.bgmv_read_once_bytes(wl, [c], False) == sb + eb
    assert B.bgmv_read_once_bytes(wl, [c], True) == sb + eb - 2 * R * n_act
