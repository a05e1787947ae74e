"""GPU tests of the MoE paths' device-side rules and of their byte identity
with one-row calls ("Module moe_lora_grouped": moe_lora_grouped_down's per-tile
early return on empty, out-of-range or unadapted expert spans, and
moe_lora_gather_bgmv; "Function apply_lora_bgmv": a batched call is
byte-identical to row-by-row calls, and the GRAPH-SAFE paragraph: fixed
buffers whose routing contents change between replays).

Every case goes through librld.so's C ABI on cuda:0.
"""
import numpy as np
import pytest
import torch

import oracle as O
import routed_lora_delta_amd as R
import workloads as W
from gpu_util import (GroupedRun, Guarded, abs_sums_gather, abs_sums_grouped,
                      assert_out_close, assert_xa_close, dev_i32, oracle_gather,
                      oracle_grouped_window, require_gpu, run_gather, say, shrink_depth)
from routed_lora_delta_amd.pool import MoeRoute, from_device_u16, grouped_windows, to_device_u16

pytestmark = pytest.mark.gpu

NEG0 = 0x8000   # -0.0: a fold with a zero delta would turn it into +0.0
QNAN = 0x7FA1   # a NaN payload that an fp32 round trip through a fold would change


def _small(seed=4, **kw):
    args = dict(num_tokens=300, top_k=4, num_experts=16, hidden=520, inter=264, max_loras=3,
                n_adapted=12, ranks=(8, 16, 32), max_rank=32, cap=256)
    args.update(kw)
    return W.moe_grouped(seed, **args)


def _corrupt_tokens(wl, rng):
    """sorted_token_ids with entries past num_tokens and below zero at rows that
    would otherwise fold; returns (new map, the corrupted rows)."""
    stid = wl.sorted_token_ids.copy()
    rows = np.sort(rng.choice(wl.te, size=24, replace=False))
    bad = [wl.num_tokens, wl.num_tokens + 7, 10 ** 6, -1, -5, -(10 ** 6)]
    for i, r in enumerate(rows):
        stid[r] = bad[i % len(bad)]
    return stid, rows


def _mark_rows(p, rows, n_out):
    """Base values of the given sorted rows set to -0.0 and a NaN payload, so
    that a read-modify-write with a zero delta shows."""
    b = p.base.reshape(-1, n_out)
    for i, r in enumerate(rows):
        b[r, 0::2] = NEG0
        b[r, 1::2] = QNAN if i % 2 else NEG0


GROUPED_CASES = {
    # name: (projection, hidden, inter, max_rank)
    "down_one_chunk": ("down", 520, 264, 32),      # k_in 264, four-wave kernel, one chunk
    "down_k_split": ("down", 520, 1544, 48),       # k_in 1544 at rank 48: chunks of 512
    "gate_fused": ("gate", 2048, 264, 32),         # wide shrink and fold in one kernel
    "gate_wide_expand": ("gate", 2048, 1032, 32),  # wide shrink, separate expand (n_out 1032)
}


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("adapter_mode", ["row_adapter", "null"])
@pytest.mark.parametrize("case", list(GROUPED_CASES))
def test_grouped_invalid_tokens_and_short_table(case, adapter_mode, separate):
    """sorted_token_ids entries >= num_tokens or < 0, with the x gather (gate)
    and without it (down), with and without row_adapter, and an offsets array
    that lists 16 experts over a route table of 12: rows with a bad token and
    rows of experts 12..15 are base rows -- output bit-identical (their -0.0
    and NaN base values included), xa zero -- and the rest meets the oracle."""
    dev = require_gpu()
    proj, hidden, inter, max_rank = GROUPED_CASES[case]
    wl = _small(seed=31, hidden=hidden, inter=inter, max_rank=max_rank,
                ranks=(8, max_rank), projections=(proj,),
                max_loras=1 if adapter_mode == "null" else 3)
    p = wl.projections[0]
    ra = "wl" if adapter_mode == "row_adapter" else None
    rng = np.random.default_rng(32)
    stid, bad_rows = _corrupt_tokens(wl, rng)
    table = wl.num_experts - 4
    past = np.flatnonzero(wl.sorted_expert >= table)
    _mark_rows(p, np.concatenate([bad_rows, past[::7]]), p.n_out)
    say(f"case: grouped invalid values {case} {adapter_mode} separate={separate} "
        f"k_in={p.k_in} n_out={p.n_out}")
    run = GroupedRun(wl, p, dev, cap=wl.cap, row_adapter=ra, stid=stid, table_experts=table)
    xas = run.run(separate=separate)
    out_g = run.base.body()
    base = p.base.ravel().copy()
    for (lo, hi), xa_g in zip(grouped_windows(wl.te, wl.cap), xas):
        xa_o, base = oracle_grouped_window(wl, p, lo, hi, base, ra, stid=stid,
                                           table_experts=table)
        assert_xa_close(xa_g, xa_o, f"invalid {case} xa [{lo},{hi})",
                        lambda lo=lo, hi=hi: abs_sums_grouped(wl, p, lo, hi, ra, stid=stid),
                        shrink_depth("grouped", p.k_in, wl.max_rank))
        skip = [r - lo for r in list(bad_rows) + list(past) if lo <= r < hi]
        assert np.all(xa_g[skip] == 0), f"{case}: xa of a skipped row is not zero"
    assert_out_close(out_g, base, f"invalid {case} out")
    o2, b2 = out_g.reshape(wl.te, p.n_out), p.base.reshape(wl.te, p.n_out)
    for r in list(bad_rows) + list(past):
        assert np.array_equal(o2[r], b2[r]), f"{case}: skipped row {r} was written"
    untouched = (base == p.base.ravel()).reshape(wl.te, p.n_out).all(axis=1)
    assert np.array_equal(o2[untouched], b2[untouched])


@pytest.mark.parametrize("adapter_mode", ["row_adapter", "null"])
def test_grouped_pair_invalid_tokens_and_short_table(adapter_mode):
    """The same rules through rld_moe_grouped_pair (gate and up of a window in
    one launch): bit-identical to rld_moe_grouped per projection, and both
    against the oracle."""
    dev = require_gpu()
    wl = _small(seed=33, hidden=2048, inter=264, projections=("gate", "up"), cap=700,
                max_loras=1 if adapter_mode == "null" else 3)
    ra = "wl" if adapter_mode == "row_adapter" else None
    rad = wl.row_adapter if ra == "wl" else None
    rng = np.random.default_rng(34)
    stid, bad_rows = _corrupt_tokens(wl, rng)
    table = wl.num_experts - 4
    pa, pb = wl.projections
    for p in (pa, pb):
        _mark_rows(p, bad_rows, p.n_out)
    say(f"case: grouped pair invalid values {adapter_mode}")
    ads = {p.name: [a for a in p.adapters if a.expert < table] for p in (pa, pb)}
    route_a = MoeRoute(ads[pa.name], wl.max_loras, table, wl.max_rank, pa.k_in, pa.n_out, dev)
    route_b = MoeRoute(ads[pb.name], wl.max_loras, table, wl.max_rank, pb.k_in, pb.n_out, dev)
    x = to_device_u16(pa.x.ravel(), dev)
    base_a, base_b = Guarded(pa.base.ravel(), dev), Guarded(pb.base.ravel(), dev)
    off, sd = dev_i32(wl.expert_offsets, dev), dev_i32(stid, dev)
    rd = dev_i32(rad, dev) if rad is not None else None
    xa_a = torch.zeros(wl.cap * wl.max_rank + 8, dtype=torch.int16, device=dev)
    xa_b = torch.zeros_like(xa_a)
    wins = grouped_windows(wl.te, wl.cap)
    xas = []
    for lo, hi in wins:
        R.check(R.rld_moe_grouped_pair(route_a.route, route_b.route, x, pa.k_in, 1, wl.num_tokens,
                                       off, wl.num_experts, sd, rd, lo, hi, base_a.ptr(),
                                       pa.n_out, base_b.ptr(), pb.n_out, xa_a, xa_b, wl.cap,
                                       None, 0), "rld_moe_grouped_pair")
        torch.cuda.synchronize()
        n = (hi - lo) * wl.max_rank
        xas.append((from_device_u16(xa_a)[:n].reshape(hi - lo, -1).copy(),
                    from_device_u16(xa_b)[:n].reshape(hi - lo, -1).copy()))
    for which, (p, got) in enumerate(((pa, base_a.body()), (pb, base_b.body()))):
        ref = GroupedRun(wl, p, dev, cap=wl.cap, row_adapter=ra, stid=stid, table_experts=table)
        ref_xa = ref.run()
        assert np.array_equal(got, ref.base.body()), p.name
        base = p.base.ravel().copy()
        for k, (lo, hi) in enumerate(wins):
            assert np.array_equal(xas[k][which], ref_xa[k]), (p.name, lo)
            xa_o, base = oracle_grouped_window(wl, p, lo, hi, base, ra, stid=stid,
                                               table_experts=table)
            assert_xa_close(xas[k][which], xa_o, f"pair invalid {p.name} xa [{lo},{hi})",
                            lambda lo=lo, hi=hi, p=p: abs_sums_grouped(wl, p, lo, hi, ra,
                                                                       stid=stid),
                            shrink_depth("grouped", p.k_in, wl.max_rank))
        assert_out_close(got, base, f"pair invalid {p.name} out")
        o2, b2 = got.reshape(wl.te, p.n_out), p.base.reshape(wl.te, p.n_out)
        for r in bad_rows:
            assert np.array_equal(o2[r], b2[r]), f"{p.name}: row {r} with a bad token written"
        past = wl.sorted_expert >= table
        assert np.array_equal(o2[past], b2[past]), f"{p.name}: rows of experts past the table"


def test_grouped_without_token_map():
    """sorted_token_ids may be NULL when x is not gathered and there is no
    row_adapter: every row of an adapted expert span folds on slot 0."""
    dev = require_gpu()
    wl = _small(seed=35, projections=("down",), max_loras=1)
    p = wl.projections[0]
    say("case: grouped down without sorted_token_ids")
    run = GroupedRun(wl, p, dev, cap=wl.cap, row_adapter=None, stid=None)
    for separate in (False, True):
        run.base.t.copy_(Guarded(p.base.ravel(), dev).t)
        xas = run.run(separate=separate)
        base = p.base.ravel().copy()
        for (lo, hi), xa_g in zip(grouped_windows(wl.te, wl.cap), xas):
            xa_o, base = oracle_grouped_window(wl, p, lo, hi, base, None, stid=None)
            assert_xa_close(xa_g, xa_o, f"no map xa [{lo},{hi})",
                            lambda lo=lo, hi=hi: abs_sums_grouped(wl, p, lo, hi, None),
                            shrink_depth("grouped", p.k_in, wl.max_rank))
        assert_out_close(run.base.body(), base, "no map out")


# ------------------------------------------------ batched == one-row calls ---

@pytest.mark.parametrize("adapter_mode", ["row_adapter", "null"])
def test_gather_batched_equals_single_rows(adapter_mode):
    """rld_moe_gather over the MoE decode config equals one call per flat row
    (n_rows = 1, top_k = 1, with indices, row_adapter, x, base and xa offset to
    that row), bit for bit; and the same for the two-entry-point path."""
    dev = require_gpu()
    wl = W.moe_gather() if adapter_mode == "row_adapter" else W.moe_gather(max_loras=1)
    ra = wl.row_adapter if adapter_mode == "row_adapter" else None
    say(f"case: gather batched == single rows ({adapter_mode})")
    route = MoeRoute(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank, wl.k_in, wl.n_out,
                     dev)
    x = to_device_u16(wl.x.ravel(), dev)
    idx = dev_i32(wl.indices, dev)
    rad = dev_i32(ra, dev) if ra is not None else None
    R_ = wl.max_rank
    for separate in (False, True):
        batched = run_gather(wl, dev, "wl" if ra is not None else None, separate=separate)
        base = Guarded(wl.base.ravel(), dev)
        xa = torch.zeros(wl.n_rows * R_ + 8, dtype=torch.int16, device=dev)
        for rho in range(wl.n_rows):
            t = rho // wl.top_k
            a = (route.route, x.data_ptr() + 2 * rho * wl.k_in, wl.k_in,
                 idx.data_ptr() + 4 * rho,
                 rad.data_ptr() + 4 * t if rad is not None else None, 1, 1)
            if separate:
                R.check(R.rld_moe_gather_shrink(*a, xa.data_ptr() + 2 * rho * R_), "shrink row")
                R.check(R.rld_moe_gather_expand_fold(route.route, xa.data_ptr() + 2 * rho * R_,
                                                     a[3], a[4], 1, 1,
                                                     base.ptr(rho * wl.n_out), wl.n_out),
                        "expand row")
            else:
                R.check(R.rld_moe_gather(*a, base.ptr(rho * wl.n_out), wl.n_out,
                                         xa.data_ptr() + 2 * rho * R_), "gather row")
        torch.cuda.synchronize()
        xa_rows = from_device_u16(xa)[: wl.n_rows * R_].reshape(wl.n_rows, R_)
        assert np.array_equal(xa_rows, batched[0]), f"xa, separate={separate}"
        assert np.array_equal(base.body(), batched[1]), f"out, separate={separate}"


def _one_row_windows(wl, dev, p_names, rows):
    """Each of `rows` as its own window [r, r+1): gate and up through
    rld_moe_grouped_pair, down through rld_moe_grouped_shrink then
    rld_moe_grouped_expand_fold (the step's calls), xa of row r written at row r
    of one arena (the xa pointer is offset, xa_rows_cap = 1)."""
    P = {p.name: p for p in wl.projections}
    rt = {n: MoeRoute(P[n].adapters, wl.max_loras, wl.num_experts, wl.max_rank, P[n].k_in,
                      P[n].n_out, dev) for n in p_names}
    base = {n: Guarded(P[n].base.ravel(), dev) for n in p_names}
    xa = {n: torch.zeros(wl.te * wl.max_rank + 8, dtype=torch.int16, device=dev)
          for n in p_names}
    off, stid = dev_i32(wl.expert_offsets, dev), dev_i32(wl.sorted_token_ids, dev)
    rad = dev_i32(wl.row_adapter, dev) if wl.row_adapter is not None else None
    xs = {n: to_device_u16(P[n].x.ravel(), dev) for n in p_names}
    wsb = max(R.rld_moe_grouped_workspace_bytes(1, P[n].k_in, wl.max_rank, wl.max_loras,
                                                wl.num_experts) for n in p_names)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    R_ = wl.max_rank
    for r in rows:
        if "gate" in p_names:
            g, u = P["gate"], P["up"]
            R.check(R.rld_moe_grouped_pair(rt["gate"].route, rt["up"].route, xs["gate"], g.k_in,
                                           1, wl.num_tokens, off, wl.num_experts, stid, rad,
                                           r, r + 1, base["gate"].ptr(), g.n_out,
                                           base["up"].ptr(), u.n_out,
                                           xa["gate"].data_ptr() + 2 * r * R_,
                                           xa["up"].data_ptr() + 2 * r * R_, 1, ws, wsb),
                    "pair row")
        if "down" in p_names:
            d = P["down"]
            xr = xa["down"].data_ptr() + 2 * r * R_
            R.check(R.rld_moe_grouped_shrink(rt["down"].route, xs["down"], d.k_in, d.x_gather,
                                             wl.num_tokens, off, wl.num_experts, stid, rad, r,
                                             r + 1, xr, 1, ws, wsb), "down shrink row")
            R.check(R.rld_moe_grouped_expand_fold(rt["down"].route, xr, wl.num_tokens, off,
                                                  wl.num_experts, stid, rad, r, r + 1,
                                                  base["down"].ptr(), d.n_out),
                    "down expand row")
    torch.cuda.synchronize()
    return ({n: from_device_u16(xa[n])[: wl.te * R_].reshape(wl.te, R_) for n in p_names},
            {n: base[n].body() for n in p_names})


def test_grouped_batched_equals_single_rows_full_config():
    """The MoE grouped prefill at full size: every sorted row as a one-row
    window through the step's calls equals the step's 8192-row windows, bit for
    bit (xa and output of gate, up and down)."""
    from test_gpu_parity import _grouped_step_sequence
    dev = require_gpu()
    wl = W.moe_grouped()
    say("case: grouped full config, batched windows")
    wins, xas, outs = _grouped_step_sequence(wl, dev)
    say(f"case: grouped full config, {wl.te} one-row windows x 3 projections")
    xa1, out1 = _one_row_windows(wl, dev, ("gate", "up", "down"), range(wl.te))
    for n in ("gate", "up", "down"):
        assert np.array_equal(xa1[n], np.concatenate(xas[n])), f"xa of {n}"
        assert np.array_equal(out1[n], outs[n]), f"output of {n}"


def test_grouped_batched_equals_single_rows_k_split():
    """One-row windows on the chunked kernels with a k split (down k_in 1544 at
    rank 48: fp32 partials per chunk, added by the pair's last block) equal the
    full window, bit for bit."""
    dev = require_gpu()
    wl = _small(seed=36, inter=1544, max_rank=48, ranks=(8, 48), projections=("down",),
                cap=1200)
    p = wl.projections[0]
    say(f"case: grouped k split one-row windows k_in={p.k_in}")
    full = GroupedRun(wl, p, dev, cap=wl.te)
    xa_full = full.run([(0, wl.te)], separate=True)[0]
    xa1, out1 = _one_row_windows(wl, dev, ("down",), range(wl.te))
    assert np.array_equal(xa1["down"], xa_full)
    assert np.array_equal(out1["down"], full.base.body())


# ------------------------------------------------------------ graph replay ---

def test_gather_graph_new_routing_each_replay():
    """rld_moe_gather captured once; before every replay the device indices and
    row_adapter buffers get the routing of another decode batch (including
    expert ids past the table and slots past max_loras).  Each replay meets the
    oracle for its routing, base rows bit-exact; eager work between replays."""
    dev = require_gpu()
    wl = W.moe_gather()
    say("case: gather graph, new routing per replay")
    route = MoeRoute(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank, wl.k_in, wl.n_out,
                     dev)
    x = to_device_u16(wl.x.ravel(), dev)
    base = Guarded(wl.base.ravel(), dev)
    pristine = base.t.clone()
    idx = dev_i32(wl.indices, dev)
    rad = dev_i32(wl.row_adapter, dev)
    xa = torch.zeros(wl.n_rows * wl.max_rank + 8, dtype=torch.int16, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        R.check(R.rld_moe_gather(route.route, x, wl.k_in, idx, rad, wl.top_k, wl.n_rows,
                                 base.ptr(), wl.n_out, xa, s), "captured rld_moe_gather")
    rng = np.random.default_rng(91)
    for rep in range(4):
        ind = np.stack([rng.choice(wl.num_experts, size=wl.top_k, replace=False)
                        for _ in range(wl.num_tokens)]).astype(np.int32).ravel()
        ind[rng.choice(wl.n_rows, 5, replace=False)] = [-1, wl.num_experts, 999, -50, 128]
        radp = rng.integers(-2, wl.max_loras + 2, size=wl.num_tokens).astype(np.int32)
        idx.copy_(torch.from_numpy(ind))
        rad.copy_(torch.from_numpy(radp))
        base.t.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wl2 = W.MoeGatherWorkload(**{**wl.__dict__, "indices": ind, "row_adapter": radp})
        xa_o, out_o = oracle_gather(wl2)
        xa_g = from_device_u16(xa)[: wl.n_rows * wl.max_rank].reshape(wl.n_rows, wl.max_rank)
        assert_xa_close(xa_g, xa_o, f"gather replay {rep} xa", abs_sums_gather(wl2),
                        shrink_depth("gather", wl.k_in, wl.max_rank))
        out_g = base.body()
        assert_out_close(out_g, out_o, f"gather replay {rep} out")
        inactive = np.all(xa_o == 0, axis=1)
        b2 = wl.base.reshape(wl.n_rows, wl.n_out)
        assert np.array_equal(out_g.reshape(wl.n_rows, wl.n_out)[inactive], b2[inactive])
        assert np.all(xa_g[inactive] == 0)
        _ = torch.ones(1 << 20, device=dev).sum().item()  # eager work between replays


# ------------------------------------------------------------ row strides --
#
# Every entry point takes element row strides for x and for the folded output
# ("Function apply_lora_bgmv", STRIDES paragraph): a fold may land inside a
# wider row.  The MoE folds read x rows at x + row * x_row_stride and fold
# [0, n_out) of base_out + row * out_row_stride; the rest of each row is left
# untouched.

def _strided(rows_bits, width, stride, rng):
    """rows_bits [rows, width] inside a buffer of rows x stride BF16 values whose
    gaps hold other values (finite, so that a stray read would show)."""
    rows = rows_bits.reshape(-1, width)
    buf = (rng.integers(0x3C00, 0x4000, size=(rows.shape[0], stride))).astype(np.uint16)
    buf[:, :width] = rows
    return buf


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("rank", [16, 24])
def test_gather_strided_rows(rank, separate):
    """The gather fold with x rows of stride k_in + 40 and outputs of stride
    n_out + 24 (the three-round path at rank 16, the general one at rank 24):
    xa and the folded [0, n_out) of every row meet the oracle's strided fold;
    the rest of each output row is bit-exact."""
    dev = require_gpu()
    wl = W.moe_gather(num_tokens=13, top_k=6, num_experts=40, k_in=1000, n_out=520, max_loras=5,
                      n_adapted=25, ranks=(8, rank), max_rank=rank)
    rng = np.random.default_rng(41)
    xs, os_ = wl.k_in + 40, wl.n_out + 24
    xbuf = _strided(wl.x, wl.k_in, xs, rng)
    bbuf = _strided(wl.base, wl.n_out, os_, rng)
    say(f"case: gather strided rows rank {rank} separate={separate}")
    route = MoeRoute(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank, wl.k_in, wl.n_out,
                     dev)
    x = to_device_u16(xbuf.ravel(), dev)
    base = Guarded(bbuf.ravel(), dev)
    idx = dev_i32(wl.indices, dev)
    rad = dev_i32(wl.row_adapter, dev)
    xa = torch.zeros(wl.n_rows * wl.max_rank + 8, dtype=torch.int16, device=dev)
    if separate:
        R.check(R.rld_moe_gather_shrink(route.route, x, xs, idx, rad, wl.top_k, wl.n_rows, xa),
                "rld_moe_gather_shrink")
        R.check(R.rld_moe_gather_expand_fold(route.route, xa, idx, rad, wl.top_k, wl.n_rows,
                                             base.ptr(), os_), "rld_moe_gather_expand_fold")
    else:
        R.check(R.rld_moe_gather(route.route, x, xs, idx, rad, wl.top_k, wl.n_rows, base.ptr(),
                                 os_, xa), "rld_moe_gather")
    torch.cuda.synchronize()
    xa_g = from_device_u16(xa)[: wl.n_rows * wl.max_rank].reshape(wl.n_rows, wl.max_rank)
    out_g = base.body().reshape(wl.n_rows, os_)
    pairs = O.pack_expert_pairs(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank)
    xa_o, out_o = O.moe_gather(pairs, wl.num_experts, wl.k_in, wl.n_out, wl.max_rank,
                               xbuf.ravel(), xs, wl.indices, wl.row_adapter, wl.top_k, wl.n_rows,
                               bbuf.ravel(), os_)
    out_o = out_o.reshape(wl.n_rows, os_)
    assert_xa_close(xa_g, xa_o, "strided gather xa", abs_sums_gather(wl),
                    shrink_depth("gather", wl.k_in, wl.max_rank))
    assert_out_close(out_g[:, :wl.n_out].ravel(), out_o[:, :wl.n_out].ravel(),
                     "strided gather out")
    assert np.array_equal(out_g[:, wl.n_out:], bbuf[:, wl.n_out:]), "row gaps changed"


@pytest.mark.parametrize("call", ["fold", "separate", "pair"])
def test_grouped_strided_rows(call):
    """The grouped fold with strided rows: gate (x gathered by token from rows of
    stride hidden + 24) and down (sorted x rows of stride inter + 40), outputs
    of stride n_out + 40 and n_out + 16; through rld_moe_grouped, the two stage
    entry points, or rld_moe_grouped_pair for gate and up.  xa and the folded
    [0, n_out) of every row meet the oracle's strided fold over every window;
    the rest of each output row is bit-exact."""
    dev = require_gpu()
    wl = _small(seed=9, hidden=1040, inter=264)
    rng = np.random.default_rng(43)
    byname = {p.name: p for p in wl.projections}
    names = ["gate", "up"] if call == "pair" else ["gate", "down"]
    wins = grouped_windows(wl.te, wl.cap)
    off = dev_i32(wl.expert_offsets, dev)
    stid = dev_i32(wl.sorted_token_ids, dev)
    rad = dev_i32(wl.row_adapter, dev)
    st = {}
    for name in names:
        p = byname[name]
        xs = p.k_in + (24 if p.x_gather else 40)
        os_ = p.n_out + (40 if name != "up" else 16)
        xbuf = _strided(p.x, p.k_in, xs, rng)
        bbuf = _strided(p.base, p.n_out, os_, rng)
        route = MoeRoute(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank, p.k_in, p.n_out,
                         dev)
        wsb = R.rld_moe_grouped_workspace_bytes(wl.cap, p.k_in, wl.max_rank, wl.max_loras,
                                                wl.num_experts)
        st[name] = dict(p=p, xs=xs, os=os_, xbuf=xbuf, bbuf=bbuf, route=route,
                        x=to_device_u16(xbuf.ravel(), dev), base=Guarded(bbuf.ravel(), dev),
                        xa=torch.zeros(wl.cap * wl.max_rank + 8, dtype=torch.int16, device=dev),
                        ws=torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev), wsb=wsb,
                        xas=[])
    say(f"case: grouped strided rows via {call}")

    def keep_xa(s, lo, hi):
        torch.cuda.synchronize()
        s["xas"].append(from_device_u16(s["xa"])[: (hi - lo) * wl.max_rank]
                        .reshape(hi - lo, wl.max_rank).copy())

    for lo, hi in wins:
        if call == "pair":
            a, b = st["gate"], st["up"]
            R.check(R.rld_moe_grouped_pair(a["route"].route, b["route"].route, a["x"], a["xs"],
                                           a["p"].x_gather, wl.num_tokens, off, wl.num_experts,
                                           stid, rad, lo, hi, a["base"].ptr(), a["os"],
                                           b["base"].ptr(), b["os"], a["xa"], b["xa"], wl.cap,
                                           a["ws"], a["wsb"]), "rld_moe_grouped_pair")
            keep_xa(a, lo, hi)
            keep_xa(b, lo, hi)
            continue
        for s in st.values():
            p = s["p"]
            if call == "separate":
                R.check(R.rld_moe_grouped_shrink(s["route"].route, s["x"], s["xs"], p.x_gather,
                                                 wl.num_tokens, off, wl.num_experts, stid, rad,
                                                 lo, hi, s["xa"], wl.cap, s["ws"], s["wsb"]),
                        "rld_moe_grouped_shrink")
                R.check(R.rld_moe_grouped_expand_fold(s["route"].route, s["xa"], wl.num_tokens,
                                                      off, wl.num_experts, stid, rad, lo, hi,
                                                      s["base"].ptr(), s["os"]),
                        "rld_moe_grouped_expand_fold")
            else:
                R.check(R.rld_moe_grouped(s["route"].route, s["x"], s["xs"], p.x_gather,
                                          wl.num_tokens, off, wl.num_experts, stid, rad, lo, hi,
                                          s["base"].ptr(), s["os"], s["xa"], wl.cap, s["ws"],
                                          s["wsb"]), "rld_moe_grouped")
            keep_xa(s, lo, hi)
    torch.cuda.synchronize()
    for name, s in st.items():
        p = s["p"]
        pairs = O.pack_expert_pairs(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank)
        out_o = s["bbuf"].ravel()
        for (lo, hi), xa_g in zip(wins, s["xas"]):
            xa_o, out_o = O.moe_grouped(pairs, wl.num_experts, p.k_in, p.n_out, wl.max_rank,
                                        s["xbuf"].ravel(), s["xs"], p.x_gather, wl.num_tokens,
                                        wl.expert_offsets, wl.sorted_token_ids, wl.row_adapter,
                                        lo, hi, out_o, s["os"])
            assert_xa_close(xa_g, xa_o, f"strided {name} xa [{lo},{hi})",
                            abs_sums_grouped(wl, p, lo, hi),
                            shrink_depth("grouped", p.k_in, wl.max_rank))
        out_g = s["base"].body().reshape(wl.te, s["os"])
        out_o = out_o.reshape(wl.te, s["os"])
        assert_out_close(out_g[:, :p.n_out].ravel(), out_o[:, :p.n_out].ravel(),
                         f"strided {name} out")
        assert np.array_equal(out_g[:, p.n_out:], s["bbuf"][:, p.n_out:]), f"{name}: row gaps"
