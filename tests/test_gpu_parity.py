"""GPU parity of every hot-path entry point against the CPU oracle.

Every case calls librld.so through the C ABI on cuda:0 and compares, element by
element, with the oracle on the same seeded inputs: xa within 1 BF16 ulp,
folded outputs within 2 BF16 ulp or 1e-3 absolute, and bit-exact everything
that is routing: base rows, xa rows of base rows, regions outside [0, n_out)
of each row, guard bands around every output buffer.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import routed_lora_delta_amd as R
import workloads as W
from gpu_util import (BgmvRun, GroupedRun, Guarded, abs_sums_bgmv, abs_sums_gather,
                      abs_sums_grouped, abs_sums_rows, assert_out_close, assert_xa_close,
                      compare_bgmv, dev_i32,
                      expand_depth, oracle_gather, oracle_grouped_window, require_gpu,
                      run_gather, say, shrink_depth)
from routed_lora_delta_amd.pool import (DenseRoute, SinglePair, from_device_u16, grouped_windows,
                                        to_device_u16)

pytestmark = pytest.mark.gpu


def _base_rows_xa_zero(wl, run):
    for i, c in enumerate(wl.calls):
        xa = run.xa_by_call[i]
        for r in range(wl.n):
            s = int(wl.seq_slot[r])
            if not (0 <= s < c.max_loras and any(a.slot == s for a in c.adapters)):
                assert np.all(xa[r] == 0), f"xa row {r} of a base row is not zero"


# ------------------------------------------------------------------- BGMV ----

def test_bgmv_tiny_config():
    dev = require_gpu()
    wl = W.bgmv_tiny()
    say(f"case: {wl.name} seq={wl.seq_slot.tolist()}")
    run = BgmvRun(wl, dev)
    run.run_all()
    compare_bgmv(run, wl.name)
    _base_rows_xa_zero(wl, run)


BGMV_SHAPES = [
    # n, k_in, n_out, max_rank, max_loras, ranks, absent slots
    (1, 256, 256, 8, 2, (4, 8), ()),
    (5, 1000, 264, 16, 3, (8, 16), ()),
    (37, 4096, 1032, 16, 16, (8, 16), (3, 7)),
    (70, 2056, 520, 24, 5, (8, 24), (1,)),
    (130, 12288, 4096, 64, 8, (8, 16, 32, 64), ()),
    (300, 512, 768, 128, 4, (64, 128), ()),
    (600, 1536, 264, 32, 40, (16, 32), (0, 39)),
    (1200, 256, 264, 16, 2, (8, 16), ()),
    (1400, 1024, 264, 16, 2, (8, 16), ()),  # k split with > 512 rows per slot
    # (column tiles x slots) grids above 768 take the lean expand item: rank
    # steps 1, 2 (one half masked at rank 48) and 4, more than 256 rows, a
    # ragged last column tile
    (700, 1024, 8192, 64, 32, (8, 16, 32, 64), (5,)),
    (90, 512, 6144, 48, 40, (16, 48), ()),
    (64, 256, 4096, 128, 64, (64, 128), ()),
    (257, 768, 3336, 8, 80, (4, 8), (2,)),
    # the classic expand's four row parts (n > 64): a slot of more than 128 of
    # 256 rows (the general path, part 0 alone) beside one of 65-128 rows
    # (three or four parts), and one slot holding every active row of 128
    (256, 1024, 1032, 64, 2, (64,), ()),
    (128, 2048, 1032, 32, 1, (32,), ()),
    # a thousand slots, most of them without a row of the batch
    (64, 1024, 264, 16, 1000, (8, 16), ()),
]


@pytest.mark.parametrize("shape", BGMV_SHAPES, ids=lambda s: f"n{s[0]}k{s[1]}o{s[2]}r{s[3]}")
def test_bgmv_shapes(shape):
    dev = require_gpu()
    n, k_in, n_out, R_, L, ranks, absent = shape
    wl = W.bgmv_custom(n, n, k_in, n_out, R_, L, ranks, base_frac=0.1, absent=absent,
                       zipf=1.1 if n > 100 else None)
    say(f"case: bgmv {shape}")
    run = BgmvRun(wl, dev)
    run.run_all()
    compare_bgmv(run, str(shape))
    _base_rows_xa_zero(wl, run)


def test_bgmv_gated_q_fold():
    """A gated model's q projection writes rows of interleaved [Q | gate] values;
    the q pair's delta folds over the whole q_proj width, at offset 0 of that
    raw row, before the Q and gate values are de-interleaved (Qwen3 attention
    LoRA weights page, the q pair's fold site).  The q adapter's B therefore has
    2 * 4096 rows here, and the row stride is that width."""
    dev = require_gpu()
    n, k_in, q_width = 48, 4096, 2 * 4096
    wl = W.bgmv_custom(12, n, k_in, q_width, 16, 16, (8, 16), base_frac=0.1,
                       out_row_stride=q_width, out_offset=0)
    say("case: gated q fold over the whole [Q|gate] row")
    run = BgmvRun(wl, dev)
    run.run_all()
    compare_bgmv(run, "gated q")


def test_bgmv_partial_row_fold():
    """A fold that covers the first half of each output row (offset 0, row
    stride 2 * n_out): the other half of every row stays bit-identical
    (compare_bgmv checks every element of the buffer outside the folded
    regions; the assertion below restates it for the second halves)."""
    dev = require_gpu()
    n, k_in, n_out = 48, 4096, 4096
    wl = W.bgmv_custom(12, n, k_in, n_out, 16, 16, (8, 16), base_frac=0.1,
                       out_row_stride=2 * n_out, out_offset=0)
    say("case: fold into the first half of each row")
    run = BgmvRun(wl, dev)
    run.run_all()
    compare_bgmv(run, "partial row")
    out = run.outputs()["out"].reshape(n, 2 * n_out)
    assert np.array_equal(out[:, n_out:], wl.buffers["out"].reshape(n, 2 * n_out)[:, n_out:])


def test_bgmv_out_of_range_slots_and_missing_tables():
    """Slots >= max_loras, negative slots and slots whose A or B entry is 0
    leave their rows untouched and write zero xa."""
    dev = require_gpu()
    wl = W.bgmv_custom(9, 12, 520, 264, 16, 4, (16,), base_frac=0.0)
    wl.seq_slot[:] = np.array([0, 1, 2, 3, 4, 77, -1, -9, 1, 2, 3, 0], np.int32)
    say("case: bgmv out-of-range slots / zeroed table entries")
    run = BgmvRun(wl, dev)
    run.routes[0].set_table_entry(2, b_addr=0)  # slot 2: B entry 0 -> base only
    run.routes[0].set_table_entry(3, a_addr=0)  # slot 3: A entry 0 -> base only
    run.run_all()
    c = wl.calls[0]
    slots = O.pack_slots(c.adapters, c.max_loras, c.max_rank)
    slots[2] = O.SlotWeights(slots[2].A, None, slots[2].scale)
    slots[3] = O.SlotWeights(None, slots[3].B, slots[3].scale)
    xa_o, out_o = O.bgmv(slots, c.k_in, c.n_out, c.max_rank, wl.buffers["x"], c.x_row_stride,
                         wl.seq_slot, wl.n, wl.buffers["out"], 0, c.n_out)
    out_g = run.outputs()["out"]
    assert_xa_close(run.xa_by_call[0], xa_o, "xa", abs_sums_bgmv(wl, c),
                    shrink_depth("bgmv", c.k_in, c.max_rank))
    assert_out_close(out_g, out_o, "out")
    for r, s in enumerate(wl.seq_slot):
        row = slice(r * c.n_out, (r + 1) * c.n_out)
        if s not in (0, 1):
            assert np.array_equal(out_g[row], wl.buffers["out"][row])
            assert np.all(run.xa_by_call[0][r] == 0)


@pytest.mark.parametrize("case", ["attn_qkv", "ffn_gate_up", "small_one_chunk", "four_routes"])
def test_bgmv_multi_equals_separate_calls(case):
    """rld_bgmv_multi over routes that read the same rows is bit-identical, xa
    and every output buffer, to rld_bgmv on each route alone: q, k and v of
    the attention decode (the K and V folds inside [Q|K|V] rows), gate and up
    of the FFN decode (k split, rank 64), a one-chunk shape, and the most
    routes a call takes (four, k split at rank 32, different n_out and
    max_loras)."""
    dev = require_gpu()
    if case == "attn_qkv":
        wl, mods = W.bgmv_attn_decode(), ("q", "k", "v")
    elif case == "ffn_gate_up":
        wl, mods = W.bgmv_ffn_decode(), ("gate", "up")
    else:
        # two routes with different n_out and max_loras over one x and seq_slot
        a = W.bgmv_custom(5, 40, 256, 264, 16, 4, (8, 16), base_frac=0.2, zipf=1.1)
        b = W.bgmv_custom(6, 40, 256, 136, 16, 6, (8, 16))
        c2 = dataclasses.replace(b.calls[0], module="proj2", out_buf="out2")
        wl = W.BgmvWorkload("two routes", a.n, a.seq_slot,
                            {**a.buffers, "out2": b.buffers["out"]}, [a.calls[0], c2])
        mods = None
    if case == "four_routes":
        parts = [W.bgmv_custom(s, 90, 1024, n_out, 32, L, (8, 32), base_frac=0.1, zipf=1.1)
                 for s, n_out, L in ((5, 264, 3), (6, 136, 5), (7, 520, 4), (8, 1032, 6))]
        calls, bufs = [], {"x": parts[0].buffers["x"]}
        for j, w in enumerate(parts):
            calls.append(dataclasses.replace(w.calls[0], module=f"proj{j}", out_buf=f"out{j}"))
            bufs[f"out{j}"] = w.buffers["out"]
        wl = W.BgmvWorkload("four routes", 90, parts[0].seq_slot, bufs, calls)
    idx = [i for i, c in enumerate(wl.calls) if mods is None or c.module in mods]
    say(f"case: bgmv multi {case} routes={len(idx)}")
    sep = BgmvRun(wl, dev)
    xa_sep = []
    for i in idx:
        sep.run_call(i)
        torch.cuda.synchronize()
        c = wl.calls[i]
        xa_sep.append(from_device_u16(sep.xa)[: wl.n * c.max_rank].reshape(wl.n, c.max_rank))
    multi = BgmvRun(wl, dev)
    xa_multi = multi.run_multi(idx)
    for i, a, b in zip(idx, xa_sep, xa_multi):
        assert np.array_equal(a, b), f"xa of {wl.calls[i].module}"
    o_sep, o_multi = sep.outputs(), multi.outputs()
    for k in o_sep:
        assert np.array_equal(o_sep[k], o_multi[k]), f"buffer {k}"


ONEPASS_CASES = [
    # n, k_in, n_out, max_rank, max_loras, ranks, absent slots, zipf, seq out of range
    (64, 4096, 4096, 16, 16, (8, 16), (), None, False),      # attention q / o shape
    (37, 1000, 520, 16, 16, (8, 16), (3, 7), None, True),    # 4 chunks, a partial last step
    (5, 200, 264, 8, 3, (4, 8), (), None, False),            # one chunk shorter than 256
    (256, 4096, 1032, 16, 16, (8, 16), (), 1.1, False),      # busy slots: several 16-row batches
    (1, 256, 256, 8, 2, (4, 8), (), None, False),
]


@pytest.mark.parametrize("case", ONEPASS_CASES, ids=lambda c: f"n{c[0]}k{c[1]}o{c[2]}r{c[3]}")
def test_bgmv_onepass_equals_three_launches(case):
    """At max_rank <= 16 and decode batch sizes rld_bgmv is one launch whose
    blocks recompute their slot's xa in the summation order of the k-split
    shrink and its chunk reduce; its xa and folded outputs are bit-identical
    to rld_bgmv_shrink + rld_bgmv_expand_fold (three launches), base rows,
    absent slots and slots past max_loras included."""
    dev = require_gpu()
    n, k_in, n_out, R_, L, ranks, absent, zipf, oob = case
    wl = W.bgmv_custom(21, n, k_in, n_out, R_, L, ranks, base_frac=0.1, absent=absent, zipf=zipf)
    if oob:
        seq = wl.seq_slot.copy()
        seq[::9] = L + 3  # past the table: base rows
        wl = dataclasses.replace(wl, seq_slot=seq)
    say(f"case: one-pass vs three launches {case}")
    one, three = BgmvRun(wl, dev), BgmvRun(wl, dev)
    assert R.rld_bgmv_launches(one.routes[0].route, n) == 1
    one.run_all()
    three.run_all(two_stage=True)
    assert np.array_equal(one.xa_by_call[0], three.xa_by_call[0]), "xa"
    assert np.array_equal(one.outputs()["out"], three.outputs()["out"]), "folded outputs"
    compare_bgmv(one, str(case))
    _base_rows_xa_zero(wl, one)


def test_bgmv_onepass_multi_equals_three_launches():
    """rld_bgmv_multi over the attention decode's q, k and v (one launch in the
    one-pass form) against each route through the two stage entry points."""
    dev = require_gpu()
    wl = W.bgmv_attn_decode()
    idx = [i for i, c in enumerate(wl.calls) if c.module in ("q", "k", "v")]
    say("case: one-pass multi q/k/v vs three launches per route")
    multi = BgmvRun(wl, dev)
    assert R.rld_bgmv_launches([multi.routes[i].route for i in idx], wl.n) == 1
    xa_multi = multi.run_multi(idx)
    three = BgmvRun(wl, dev)
    for i, xm in zip(idx, xa_multi):
        three.run_call_two_stage(i)
        torch.cuda.synchronize()
        c = wl.calls[i]
        xt = from_device_u16(three.xa)[: wl.n * c.max_rank].reshape(wl.n, c.max_rank)
        assert np.array_equal(xm, xt), f"xa of {c.module}"
    o_m, o_t = multi.outputs(), three.outputs()
    for k in o_m:
        assert np.array_equal(o_m[k], o_t[k]), f"buffer {k}"


def test_bgmv_batched_equals_single_rows():
    """BGMV over n rows is bit-identical to n calls with n = 1 on offset
    pointers (xa and folded output)."""
    dev = require_gpu()
    for n, k_in, n_out, R_, ranks in ((64, 4096, 1024, 16, (8, 16)), (200, 12288, 520, 64, (8, 64))):
        wl = W.bgmv_custom(11, n, k_in, n_out, R_, 8, ranks, base_frac=0.1, zipf=1.1)
        say(f"case: batched vs single rows n={n} k_in={k_in}")
        run = BgmvRun(wl, dev)
        run.run_all()
        batched_out = run.outputs()["out"]
        batched_xa = run.xa_by_call[0]
        c = wl.calls[0]
        single = BgmvRun(wl, dev)
        xa1 = torch.zeros(R_ + 8, dtype=torch.int16, device=dev)
        ws_b = R.rld_bgmv_workspace_bytes(1, k_in, R_, 8)
        ws1 = torch.zeros(max(ws_b, 16) // 4 + 4, dtype=torch.float32, device=dev)
        xas = []
        for i in range(n):
            R.check(R.rld_bgmv(single.routes[0].route, single.bufs["x"].ptr(i * c.x_row_stride),
                               c.x_row_stride, single.seq.data_ptr() + 4 * i, 1,
                               single.bufs["out"].ptr(i * c.out_row_stride), c.out_row_stride,
                               xa1, ws1, ws_b), "single-row bgmv")
            torch.cuda.synchronize()
            xas.append(from_device_u16(xa1)[:R_].copy())
        assert np.array_equal(np.stack(xas), batched_xa)
        assert np.array_equal(single.outputs()["out"], batched_out)


def test_bgmv_graph_replays():
    """rld_bgmv captured in a HIP graph (k split over 8 chunks: shrink, chunk
    reduce and expand): every replay, with eager work and synchronisations
    between replays, gives the eager call's bits."""
    dev = require_gpu()
    wl = W.bgmv_custom(22, 256, 4096, 2048, 64, 16, (16, 64), base_frac=0.05, zipf=1.1)
    say("case: graph replays")
    eager = BgmvRun(wl, dev)
    eager.run_all(keep_xa=False)
    want = eager.outputs()["out"]
    run = BgmvRun(wl, dev)
    pristine = run.bufs["out"].t.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        run.run_call(0, stream=s)
    for rep in range(4):
        run.bufs["out"].t.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(run.outputs()["out"], want), f"replay {rep}"
        _ = torch.ones(1 << 20, device=dev).sum().item()  # eager work between replays


def test_bgmv_delta_stage():
    """The expand's delta (observed with scale 1 and base 0) is within 1 ulp of
    the oracle's delta computed from the GPU's own xa."""
    dev = require_gpu()
    n, k_in, n_out, R_ = 50, 4096, 4096, 16
    rng = W.rng_for(5, salt=3)
    ads = [W.make_adapter(rng, s, r, k_in, n_out, float(r), False) for s, r in enumerate((16, 8, 12))]
    seq = rng.integers(-1, 3, size=n).astype(np.int32)
    x = W._normal(rng, (n, k_in)).ravel()
    zero = np.zeros(n * n_out, np.uint16)
    wl = W.BgmvWorkload("delta", n, seq, {"x": x, "out": zero},
                        [W.BgmvCall("p", k_in, n_out, R_, 3, ads, "x", k_in, "out", 0, n_out)])
    say("case: delta stage")
    run = BgmvRun(wl, dev)
    run.run_all()
    xa_g = run.xa_by_call[0]
    delta_g = run.outputs()["out"].reshape(n, n_out)
    slots = O.pack_slots(ads, 3, R_)
    for i in range(n):
        s = int(seq[i])
        if s < 0:
            assert np.all(delta_g[i] == 0)
            continue
        d_o = O.round_bf16(slots[s].b64() @ O.bf16_to_f64(xa_g[i]))
        assert_xa_close(delta_g[i], d_o, f"delta row {i}",
                        abs_sums_rows(xa_g[i][None], slots[s].B)[0], expand_depth("bgmv", R_))


# each full-size configuration at its own seed and at a second one
@pytest.mark.parametrize("seed_index", [1, 101], ids=lambda v: f"seed{v}")
def test_bgmv_attn_decode_config(seed_index):
    """Qwen3-8B attention side: q contiguous, k/v folded inside [Q|K|V] rows."""
    dev = require_gpu()
    wl = W.bgmv_attn_decode(seed_index)
    say(f"case: {wl.name}")
    run = BgmvRun(wl, dev)
    run.run_all()
    compare_bgmv(run, wl.name)
    _base_rows_xa_zero(wl, run)


@pytest.mark.parametrize("seed_index", [2, 102], ids=lambda v: f"seed{v}")
def test_bgmv_ffn_decode_config(seed_index):
    dev = require_gpu()
    wl = W.bgmv_ffn_decode(seed_index)
    say(f"case: {wl.name}")
    run = BgmvRun(wl, dev)
    run.run_all()
    compare_bgmv(run, wl.name)
    _base_rows_xa_zero(wl, run)


def test_bgmv_shared_workspace_second_pass():
    """One workspace shared by calls of different shapes (gate/up split k_in in
    4 chunks, down in 12), used for a second pass after the first: the second
    pass (outputs restored to the base values first, now through the separate
    shrink and expand entry points) still meets the oracle, so no call's scratch
    disturbs another's."""
    dev = require_gpu()
    wl = W.bgmv_ffn_decode()
    say(f"case: shared workspace, second pass, {wl.name}")
    run = BgmvRun(wl, dev)
    pristine = {k: b.t.clone() for k, b in run.bufs.items()}
    run.run_all(keep_xa=False)
    for k, b in run.bufs.items():
        b.t.copy_(pristine[k])
    run.run_all(two_stage=True)
    compare_bgmv(run, "second pass " + wl.name)


# ------------------------------------------------------------------ gather ---

@pytest.mark.parametrize("variant", ["config", "config_seed103", "null_adapter", "ragged",
                                     "ragged_rank16", "many_pairs", "rank128"])
def test_moe_gather(variant):
    """The gather fold against the oracle: the MoE decode config, no row_adapter,
    and ragged shapes with out-of-range expert ids and slots (rank 24: the
    general kernel path; rank 16 with k_in 1000: the three-round path), and a
    route of 1152 (slot, expert) pairs at the decode shape."""
    dev = require_gpu()
    if variant == "config":
        wl = W.moe_gather()
        ra = "wl"
    elif variant == "config_seed103":
        wl = W.moe_gather(seed_index=103)
        ra = "wl"
    elif variant == "null_adapter":
        wl = W.moe_gather(num_tokens=20, top_k=4, num_experts=16, k_in=264, n_out=1032,
                          max_loras=1, n_adapted=10, max_rank=16)
        ra = None
    elif variant == "ragged":
        wl = W.moe_gather(num_tokens=13, top_k=6, num_experts=40, k_in=1000, n_out=520,
                          max_loras=5, n_adapted=25, ranks=(8, 24), max_rank=24)
        wl.indices[3] = -1
        wl.indices[10] = 999
        ra = "wl"
    elif variant == "many_pairs":
        wl = W.moe_gather(num_tokens=24, top_k=8, num_experts=128, k_in=768, n_out=2048,
                          max_loras=9, n_adapted=64, max_rank=16)
        ra = "wl"
    elif variant == "rank128":  # the largest max_rank the boundary takes
        wl = W.moe_gather(num_tokens=13, top_k=6, num_experts=40, k_in=1000, n_out=520,
                          max_loras=5, n_adapted=25, ranks=(64, 128), max_rank=128)
        ra = "wl"
    else:
        wl = W.moe_gather(num_tokens=13, top_k=6, num_experts=40, k_in=1000, n_out=520,
                          max_loras=5, n_adapted=25, ranks=(8, 16), max_rank=16)
        wl.indices[3] = -1
        wl.indices[10] = 999
        wl.row_adapter[2] = 7    # slot past max_loras: the token's rows stay base rows
        wl.row_adapter[5] = -1
        ra = "wl"
    say(f"case: gather {variant} {wl.name}")
    xa_g, out_g = run_gather(wl, dev, ra)
    xa_o, out_o = oracle_gather(wl, ra)
    assert_xa_close(xa_g, xa_o, "gather xa", abs_sums_gather(wl, ra),
                    shrink_depth("gather", wl.k_in, wl.max_rank))
    assert_out_close(out_g, out_o, "gather out")
    inactive = np.all(xa_o == 0, axis=1)
    base2 = wl.base.reshape(wl.n_rows, wl.n_out)
    assert np.array_equal(out_g.reshape(wl.n_rows, wl.n_out)[inactive], base2[inactive])
    assert np.all(xa_g[inactive] == 0)
    # the one-launch combined call and the two entry points agree bit for bit
    xa_s, out_s = run_gather(wl, dev, ra, separate=True)
    assert np.array_equal(xa_s, xa_g)
    assert np.array_equal(out_s, out_g)


# ----------------------------------------------------------------- grouped ---

def _small_grouped(seed=4, num_tokens=300, **kw):
    args = dict(num_tokens=num_tokens, top_k=4, num_experts=16, hidden=520, inter=264,
                max_loras=3, n_adapted=12, ranks=(8, 16, 32), max_rank=32, cap=256)
    args.update(kw)
    return W.moe_grouped(seed, **args)


@pytest.mark.parametrize("proj", ["down", "gate"])
@pytest.mark.parametrize("adapter_mode", ["row_adapter", "null"])
def test_moe_grouped_small(proj, adapter_mode):
    dev = require_gpu()
    wl = _small_grouped(projections=(proj,), max_loras=1 if adapter_mode == "null" else 3)
    p = wl.projections[0]
    ra = "wl" if adapter_mode == "row_adapter" else None
    say(f"case: grouped small {proj} {adapter_mode}")
    run = GroupedRun(wl, p, dev, cap=wl.cap, row_adapter=ra)
    xas = run.run()
    out_g = run.base.body()
    base = p.base.ravel().copy()
    for (lo, hi), xa_g in zip(grouped_windows(wl.te, wl.cap), xas):
        xa_o, base = oracle_grouped_window(wl, p, lo, hi, base, ra)
        assert_xa_close(xa_g, xa_o, f"grouped xa [{lo},{hi})",
                        abs_sums_grouped(wl, p, lo, hi, ra),
                        shrink_depth("grouped", p.k_in, wl.max_rank))
        assert np.all(xa_g[np.all(xa_o == 0, axis=1)] == 0)
    assert_out_close(out_g, base, "grouped out")
    unchanged_o = base == p.base.ravel()
    # rows the oracle leaves untouched must be bit-identical on the GPU too
    rows_o = unchanged_o.reshape(wl.te, p.n_out).all(axis=1)
    assert np.array_equal(out_g.reshape(wl.te, p.n_out)[rows_o],
                          p.base.reshape(wl.te, p.n_out)[rows_o])


def test_moe_grouped_window_union_bit_exact():
    """A full-window call equals the union of its chunk windows, bit for bit,
    for caps that are and are not multiples of 64."""
    dev = require_gpu()
    wl = _small_grouped(projections=("down", "gate"), cap=2048)
    for p in wl.projections:
        say(f"case: window union {p.name}")
        full = GroupedRun(wl, p, dev, cap=wl.te)
        xa_full = full.run([(0, wl.te)])[0]
        out_full = full.base.body()
        for cap in (64, 100, 333):
            part = GroupedRun(wl, p, dev, cap=cap)
            xas = part.run(grouped_windows(wl.te, cap))
            assert np.array_equal(np.concatenate(xas), xa_full), cap
            assert np.array_equal(part.base.body(), out_full), cap


def test_moe_grouped_edge_windows():
    """Empty window (launches one m-tile, writes nothing), a single-row window,
    and a window over rows outside every expert span."""
    dev = require_gpu()
    wl = _small_grouped(projections=("down",))
    p = wl.projections[0]
    say("case: grouped edge windows")
    run = GroupedRun(wl, p, dev, cap=256)
    run.run([(50, 50)])
    assert np.array_equal(run.base.body(), p.base.ravel())
    xas = run.run([(77, 78)])
    xa_o, out_o = oracle_grouped_window(wl, p, 77, 78, p.base.ravel().copy())
    assert_xa_close(xas[0], xa_o, "single row xa", abs_sums_grouped(wl, p, 77, 78),
                    shrink_depth("grouped", p.k_in, wl.max_rank))
    assert_out_close(run.base.body(), out_o, "single row out")
    # offsets that put the last 40 rows outside every span
    off = wl.expert_offsets.copy()
    off[-1] = off[-1] - 40
    off = np.minimum(off, off[-1])
    run2 = GroupedRun(wl, p, dev, cap=wl.te)
    run2.off = dev_i32(off, dev)
    run2.run([(0, wl.te)])
    wl2 = W.MoeGroupedWorkload(**{**wl.__dict__, "expert_offsets": off})
    xa_o2, out_o2 = oracle_grouped_window(wl2, p, 0, wl.te, p.base.ravel().copy())
    assert_out_close(run2.base.body(), out_o2, "rows outside spans")
    tail = slice((wl.te - 40) * p.n_out, wl.te * p.n_out)
    assert np.array_equal(run2.base.body()[tail], p.base.ravel()[tail])


@pytest.mark.parametrize("proj,hidden", [("down", 520), ("gate", 1032)])
def test_moe_grouped_offsets_below_zero(proj, hidden):
    """Non-decreasing offsets whose first entries are negative: experts 0 and 1
    end at or below row 0 and own no row (their spans clamp to empty, never to
    a range past the window), expert 2 owns rows [0, off[3]).  The chunked
    kernels (down) and the one-launch wide fold (gate, k_in 1032)."""
    dev = require_gpu()
    wl = _small_grouped(projections=(proj,), hidden=hidden)
    p = wl.projections[0]
    say(f"case: grouped offsets below zero {proj} k_in={p.k_in}")
    off = wl.expert_offsets.copy()
    off[:3] = [-8, -4, 0]
    run = GroupedRun(wl, p, dev, cap=wl.te)
    run.off = dev_i32(off, dev)
    xas = run.run([(0, wl.te)])
    wl2 = W.MoeGroupedWorkload(**{**wl.__dict__, "expert_offsets": off,
                                  "sorted_expert": O.expert_owner(off, 0, wl.te)})
    assert wl2.sorted_expert.min() == 2
    xa_o, out_o = oracle_grouped_window(wl2, p, 0, wl.te, p.base.ravel().copy())
    assert_xa_close(xas[0], xa_o, "offsets below zero xa", abs_sums_grouped(wl2, p, 0, wl.te),
                    shrink_depth("grouped", p.k_in, wl.max_rank))
    assert_out_close(run.base.body(), out_o, "offsets below zero out")


def _grouped_step_sequence(wl, dev):
    """The MoE grouped prefill as the step issues it, window by window: the gate
    and up folds of a window in one rld_moe_grouped_pair call, then the down
    window through rld_moe_grouped_shrink and rld_moe_grouped_expand_fold.  The
    windows come from the library's own rld_grouped_windows.  Returns the
    windows, each projection's xa per window and folded output."""
    from routed_lora_delta_amd.pool import MoeRoute
    P = {p.name: p for p in wl.projections}
    g, u, d = P["gate"], P["up"], P["down"]
    rt = {p.name: MoeRoute(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank, p.k_in,
                           p.n_out, dev) for p in wl.projections}
    x_tok = to_device_u16(g.x.ravel(), dev)
    x_dn = to_device_u16(d.x.ravel(), dev)
    base = {p.name: Guarded(p.base.ravel(), dev) for p in wl.projections}
    off, stid = dev_i32(wl.expert_offsets, dev), dev_i32(wl.sorted_token_ids, dev)
    rad = dev_i32(wl.row_adapter, dev)
    wins = grouped_windows(wl.te, wl.cap)
    assert wins == O.grouped_down_windows(wl.te, wl.cap)
    xa = {n: [torch.zeros(wl.cap * wl.max_rank + 8, dtype=torch.int16, device=dev)
              for _ in wins] for n in P}
    wsb = max(R.rld_moe_grouped_workspace_bytes(wl.cap, p.k_in, wl.max_rank, wl.max_loras,
                                                wl.num_experts) for p in wl.projections)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    for k, (lo, hi) in enumerate(wins):
        R.check(R.rld_moe_grouped_pair(rt["gate"].route, rt["up"].route, x_tok, g.k_in, 1,
                                       wl.num_tokens, off, wl.num_experts, stid, rad, lo, hi,
                                       base["gate"].ptr(), g.n_out, base["up"].ptr(), u.n_out,
                                       xa["gate"][k], xa["up"][k], wl.cap, ws, wsb),
                "rld_moe_grouped_pair")
        R.check(R.rld_moe_grouped_shrink(rt["down"].route, x_dn, d.k_in, 0, wl.num_tokens, off,
                                         wl.num_experts, stid, rad, lo, hi, xa["down"][k],
                                         wl.cap, ws, wsb), "rld_moe_grouped_shrink")
        R.check(R.rld_moe_grouped_expand_fold(rt["down"].route, xa["down"][k], wl.num_tokens,
                                              off, wl.num_experts, stid, rad, lo, hi,
                                              base["down"].ptr(), d.n_out),
                "rld_moe_grouped_expand_fold")
    torch.cuda.synchronize()
    xas = {n: [from_device_u16(xa[n][k])[: (hi - lo) * wl.max_rank].reshape(hi - lo, wl.max_rank)
               for k, (lo, hi) in enumerate(wins)] for n in P}
    outs = {n: base[n].body() for n in P}
    return wins, xas, outs


@pytest.mark.parametrize("seed_index", [4, 104], ids=lambda v: f"seed{v}")
def test_moe_grouped_full_config(seed_index):
    """The MoE grouped prefill at full size (4096 tokens, top-8 of 128 experts,
    te = 32768 sorted rows in windows of 8192, down 768 -> 2048 and gate/up
    2048 -> 768 gathered, rank 32, 4 slots), through the step's own call
    sequence (the pair kernel for gate and up, shrink then expand for down):
    every xa row of every window and every output element of all three
    projections against the oracle; rows the oracle leaves untouched (slot -1,
    unadapted pair) bit-identical to the base.  The bench's step, issued
    eagerly on the same inputs, gives the same bits."""
    dev = require_gpu()
    wl = W.moe_grouped(seed_index)
    say(f"case: grouped full config seed {seed_index}, step call sequence, every row")
    wins, xas, outs = _grouped_step_sequence(wl, dev)
    for p in wl.projections:
        say(f"case: grouped full config oracle {p.name} k_in={p.k_in} n_out={p.n_out}")
        base = p.base.ravel().copy()
        for k, (lo, hi) in enumerate(wins):
            xa_o, base = oracle_grouped_window(wl, p, lo, hi, base)
            assert_xa_close(xas[p.name][k], xa_o, f"full {p.name} xa [{lo},{hi})",
                            lambda lo=lo, hi=hi, p=p: abs_sums_grouped(wl, p, lo, hi),
                            shrink_depth("grouped", p.k_in, wl.max_rank))
            assert np.all(xas[p.name][k][np.all(xa_o == 0, axis=1)] == 0)
        assert_out_close(outs[p.name], base, f"full {p.name} out")
        rows_o = (base == p.base.ravel()).reshape(wl.te, p.n_out).all(axis=1)
        assert np.array_equal(outs[p.name].reshape(wl.te, p.n_out)[rows_o],
                              p.base.reshape(wl.te, p.n_out)[rows_o]), p.name
        say(f"  {p.name}: {int((~rows_o).sum())} rows folded, {int(rows_o.sum())} untouched")
    # the bench's step on the same workload, its calls issued eagerly in order,
    # and (fresh buffers) its captured graph replayed once: each window is a
    # chain on a branch of its own (gate+up, then down, which reuses the
    # window's xa arena), so a missing edge or a shared buffer would show here
    import bench
    step = bench.Step(dev, [("grouped", wl)])
    for c in step.calls:
        R.check(c[2](), c[0])
    torch.cuda.synchronize()
    for p in wl.projections:
        got = from_device_u16(step.outputs[f"grouped.{p.name}"])[: wl.te * p.n_out]
        assert np.array_equal(got, outs[p.name]), f"bench step differs on {p.name}"
    step2 = bench.Step(dev, [("grouped", wl)])
    graph = step2.capture(range(len(step2.calls)), torch.cuda.Stream(), parallel=True)
    graph.replay()
    torch.cuda.synchronize()
    for p in wl.projections:
        got = from_device_u16(step2.outputs[f"grouped.{p.name}"])[: wl.te * p.n_out]
        assert np.array_equal(got, outs[p.name]), f"bench step graph differs on {p.name}"


def _pair_run(wl, pa, pb, dev, cap, ra="wl"):
    """Every window of the gate/up pair through rld_moe_grouped_pair: xa of
    each window and the folded outputs of both projections."""
    from routed_lora_delta_amd.pool import MoeRoute
    rad = wl.row_adapter if ra == "wl" else ra
    route_a = MoeRoute(pa.adapters, wl.max_loras, wl.num_experts, wl.max_rank, pa.k_in, pa.n_out,
                       dev)
    route_b = MoeRoute(pb.adapters, wl.max_loras, wl.num_experts, wl.max_rank, pb.k_in, pb.n_out,
                       dev)
    x = to_device_u16(pa.x.ravel(), dev)
    base_a, base_b = Guarded(pa.base.ravel(), dev), Guarded(pb.base.ravel(), dev)
    off, stid = dev_i32(wl.expert_offsets, dev), dev_i32(wl.sorted_token_ids, dev)
    rd = dev_i32(rad, dev) if rad is not None else None
    xa_a = torch.zeros(cap * wl.max_rank + 8, dtype=torch.int16, device=dev)
    xa_b = torch.zeros(cap * wl.max_rank + 8, dtype=torch.int16, device=dev)
    wsb = max(R.rld_moe_grouped_workspace_bytes(cap, p.k_in, wl.max_rank, wl.max_loras,
                                                wl.num_experts) for p in (pa, pb))
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    xas = []
    for lo, hi in grouped_windows(wl.te, cap):
        R.check(R.rld_moe_grouped_pair(route_a.route, route_b.route, x, pa.k_in, pa.x_gather,
                                       wl.num_tokens, off, wl.num_experts, stid, rd, lo, hi,
                                       base_a.ptr(), pa.n_out, base_b.ptr(), pb.n_out, xa_a,
                                       xa_b, cap, ws, wsb), "rld_moe_grouped_pair")
        torch.cuda.synchronize()
        n = (hi - lo) * wl.max_rank
        xas.append((from_device_u16(xa_a)[:n].copy(), from_device_u16(xa_b)[:n].copy()))
    return xas, base_a.body(), base_b.body()


@pytest.mark.parametrize("case", ["full", "small", "small_null", "fallback", "long", "ragged_k"])
def test_moe_grouped_pair_equals_two_calls(case):
    """rld_moe_grouped_pair on a gate/up pair equals rld_moe_grouped on each
    projection, bit for bit (every window's xa and both folded outputs).  The
    two projections adapt independent expert subsets, so some pairs fold in one
    of them only.  full: the MoE prefill at full size (one launch per window);
    small: k_in 2048 at n_out 264 (one launch); small_null: without
    row_adapter; fallback: k_in 520 (two rld_moe_grouped calls); long: pairs
    of hundreds of rows that both projections adapt (several row batches per
    item, and expert spans past one 1024-row scan segment); ragged_k: k_in
    2000, not a multiple of the waves' 128-wide k ranges."""
    dev = require_gpu()
    if case == "full":
        wl = W.moe_grouped(projections=("gate", "up"))
    elif case == "ragged_k":
        # k_in 2000: the last waves' k ranges end inside k_in or past it (masked
        # operands), every expert adapted by both projections (one pass for both)
        wl = _small_grouped(seed=11, hidden=2000, projections=("gate", "up"), cap=700,
                            n_adapted=16)
    elif case == "long":
        wl = W.moe_grouped(9, num_tokens=2400, top_k=2, num_experts=4, hidden=2048, inter=264,
                           max_loras=2, n_adapted=4, ranks=(8, 16, 32), max_rank=32,
                           cap=4800, projections=("gate", "up"))
        spans = np.diff(np.asarray(wl.expert_offsets))
        assert spans.max() > 1024, spans
    else:
        hidden = 520 if case == "fallback" else 2048
        wl = _small_grouped(seed=8, hidden=hidden, projections=("gate", "up"), cap=700,
                            max_loras=1 if case == "small_null" else 3)
    ra = None if case == "small_null" else "wl"
    pa, pb = wl.projections
    say(f"case: grouped pair {case} k_in={pa.k_in} n_out={pa.n_out} te={wl.te}")
    xas, out_a, out_b = _pair_run(wl, pa, pb, dev, wl.cap, ra)
    for p, out, which in ((pa, out_a, 0), (pb, out_b, 1)):
        run = GroupedRun(wl, p, dev, cap=wl.cap, row_adapter=ra)
        ref = run.run()
        for (lo, hi), xa_ref, xa_pair in zip(grouped_windows(wl.te, wl.cap), ref, xas):
            assert np.array_equal(xa_pair[which].reshape(xa_ref.shape), xa_ref), (p.name, lo)
        assert np.array_equal(out, run.base.body()), p.name


@pytest.mark.parametrize("max_loras,num_experts", [(5, 128), (1, 600)])
def test_moe_grouped_large_route(max_loras, num_experts):
    """Routes past the small worklist capacity (more than 512 (slot, expert)
    pairs, or 512 or more offsets entries) take the large-capacity kernels;
    both projections against the oracle, in windows."""
    dev = require_gpu()
    wl = _small_grouped(seed=6, num_tokens=400, num_experts=num_experts, max_loras=max_loras,
                        n_adapted=num_experts * 3 // 4, projections=("down", "gate"), cap=700)
    assert wl.max_loras * wl.num_experts > 512
    ra = "wl" if max_loras > 1 else None
    for p in wl.projections:
        say(f"case: grouped large route {p.name} max_loras={max_loras} E={num_experts}")
        run = GroupedRun(wl, p, dev, cap=wl.cap, row_adapter=ra)
        xas = run.run()
        base = p.base.ravel().copy()
        for (lo, hi), xa_g in zip(grouped_windows(wl.te, wl.cap), xas):
            xa_o, base = oracle_grouped_window(wl, p, lo, hi, base, ra)
            assert_xa_close(xa_g, xa_o, f"large route xa [{lo},{hi})",
                            abs_sums_grouped(wl, p, lo, hi, ra),
                            shrink_depth("grouped", p.k_in, wl.max_rank))
        assert_out_close(run.base.body(), base, "large route out")


@pytest.mark.parametrize("k_in,max_rank,proj,n_out", [
    (2048, 32, "gate", 264), (1032, 16, "gate", 264), (1544, 32, "down", 264),
    (2048, 24, "down", 264), (1160, 32, "gate", 264), (768, 32, "down", 2048),
    (264, 16, "down", 1032), (520, 64, "gate", 264), (1032, 48, "gate", 264),
    (520, 128, "gate", 264), (264, 128, "down", 1032)])
@pytest.mark.parametrize("separate", [False, True])
def test_moe_grouped_wide(k_in, max_rank, proj, n_out, separate):
    """1024 < k_in <= 2048 at max_rank <= 32: one sixteen-wave block per pair
    half covers all of k_in; k_in not a multiple of 128 leaves one wave's range
    partly past k_in and later ones wholly past it.  Through rld_moe_grouped
    (the shrink and fold in one kernel when n_out <= 768) or the two stages
    separately.  The other rows of the table take the four-wave kernels (k_in
    <= 1024: one chunk; max_rank 48 at k_in 1032: chunks of 512) and, for n_out
    above 768, the separate expand.  Pairs of up to ~100 rows (both halves,
    several batches each), windows of 333 rows against the oracle, and the full
    window bit-identical to their union."""
    dev = require_gpu()
    sizes = dict(hidden=k_in, inter=n_out) if proj == "gate" else dict(hidden=n_out, inter=k_in)
    wl = _small_grouped(seed=7, num_experts=4, n_adapted=3, max_rank=max_rank,
                        ranks=(8, max_rank), cap=333, projections=(proj,), **sizes)
    p = wl.projections[0]
    say(f"case: grouped wide {proj} k_in={k_in} n_out={n_out} max_rank={max_rank} "
        f"separate={separate}")
    run = GroupedRun(wl, p, dev, cap=wl.cap)
    xas = run.run(separate=separate)
    base = p.base.ravel().copy()
    for (lo, hi), xa_g in zip(grouped_windows(wl.te, wl.cap), xas):
        xa_o, base = oracle_grouped_window(wl, p, lo, hi, base)
        assert_xa_close(xa_g, xa_o, f"wide xa [{lo},{hi})", abs_sums_grouped(wl, p, lo, hi),
                        shrink_depth("grouped", p.k_in, wl.max_rank))
        assert np.all(xa_g[np.all(xa_o == 0, axis=1)] == 0)
    assert_out_close(run.base.body(), base, "wide out")
    full = GroupedRun(wl, p, dev, cap=wl.te)
    xa_full = full.run([(0, wl.te)], separate=not separate)[0]
    assert np.array_equal(np.concatenate(xas), xa_full)
    assert np.array_equal(full.base.body(), run.base.body())


@pytest.mark.parametrize("hidden,num_tokens", [(2056, 1200), (2048, 2400)])
@pytest.mark.parametrize("max_loras", [1, 2])
def test_moe_grouped_long_pairs(max_loras, hidden, num_tokens):
    """Pairs with hundreds of rows in one window: many row batches, and with one
    slot more than one scan segment (gate's k_in = 2056 splits into 5 chunks and
    the chunk reduce rescans the span; k_in = 2048 is the sixteen-wave kernel,
    whose segments hold 1024 rows), in one full window and in windows of 700
    rows."""
    dev = require_gpu()
    wl = W.moe_grouped(9, num_tokens=num_tokens, top_k=2, num_experts=4, hidden=hidden,
                       inter=264, max_loras=max_loras, n_adapted=4, ranks=(8, 16, 32),
                       max_rank=32, cap=2 * num_tokens, projections=("down", "gate"))
    ra = None if max_loras == 1 else "wl"
    for p in wl.projections:
        say(f"case: grouped long pairs {p.name} k_in={p.k_in} max_loras={max_loras}")
        full = GroupedRun(wl, p, dev, cap=wl.te, row_adapter=ra)
        xa_full = full.run([(0, wl.te)])[0]
        xa_o, out_o = oracle_grouped_window(wl, p, 0, wl.te, p.base.ravel().copy(), ra)
        assert_xa_close(xa_full, xa_o, f"long pairs xa {p.name}",
                        abs_sums_grouped(wl, p, 0, wl.te, ra),
                        shrink_depth("grouped", p.k_in, wl.max_rank))
        assert_out_close(full.base.body(), out_o, f"long pairs out {p.name}")
        part = GroupedRun(wl, p, dev, cap=700, row_adapter=ra)
        xas = part.run(grouped_windows(wl.te, 700))
        assert np.array_equal(np.concatenate(xas), xa_full)
        assert np.array_equal(part.base.body(), full.base.body())


def test_moe_grouped_graph_replays():
    """Every window of a projection (k split over 5 chunks, the last one ragged)
    captured in one HIP graph: each replay, with eager work and
    synchronisations between, gives the eager calls' bits, and the per-pair
    counters at the end of the workspace are back at zero after each."""
    dev = require_gpu()
    wl = _small_grouped(projections=("gate",), hidden=2056)
    p = wl.projections[0]
    say("case: grouped graph replays")
    eager = GroupedRun(wl, p, dev)
    eager.run(keep_xa=False)
    want = eager.base.body()
    run = GroupedRun(wl, p, dev)
    pristine = run.base.t.clone()
    wins = grouped_windows(wl.te, wl.cap)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        for lo, hi in wins:
            R.check(R.rld_moe_grouped(run.route.route, run.x, p.k_in, p.x_gather, wl.num_tokens,
                                      run.off, wl.num_experts, run.stid, run.rad, lo, hi,
                                      run.base.ptr(), p.n_out, run.xa, run.cap, run.ws,
                                      run.ws_bytes, s), "captured rld_moe_grouped")
    end = run.ws_bytes // 16 * 16
    npairs = wl.max_loras * wl.num_experts
    for rep in range(4):
        run.base.t.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(run.base.body(), want), f"replay {rep}"
        counters = run.ws.view(torch.int32).cpu().numpy()[(end - 16 * npairs) // 4: end // 4]
        assert np.all(counters == 0), f"replay {rep}: counters {np.flatnonzero(counters)[:8]}"
        _ = torch.ones(1 << 20, device=dev).sum().item()  # eager work between replays


def test_determinism_repeat_runs():
    dev = require_gpu()
    wl = _small_grouped(projections=("gate",))
    p = wl.projections[0]
    say("case: determinism")
    outs = []
    for _ in range(2):
        run = GroupedRun(wl, p, dev, cap=512)
        run.run()
        outs.append(run.base.body())
    assert np.array_equal(outs[0], outs[1])
    wlb = W.bgmv_custom(3, 100, 4096, 1024, 16, 8, (8, 16), zipf=1.1)
    o2 = []
    for _ in range(2):
        r = BgmvRun(wlb, dev)
        r.run_all()
        o2.append(r.outputs()["out"])
    assert np.array_equal(o2[0], o2[1])


# --------------------------------------------------------------- unrouted ---

class LoraRun:
    """Device state of one unrouted case: the pair (on slot 0 of a one-slot route,
    so the routed entry points can run on the same pool), guarded x and output
    buffers, xa and workspace."""

    def __init__(self, ad, m, k_in, n_out, max_rank, x, base, dev):
        self.sp = SinglePair(ad, max_rank, k_in, n_out, dev)
        self.m, self.k_in, self.n_out, self.R = m, k_in, n_out, max_rank
        self.x = Guarded(x, dev)
        self.base = Guarded(base, dev)
        self.xa = torch.zeros(max(m, 1) * max_rank + 8, dtype=torch.int16, device=dev)
        self.ws_bytes = R.rld_lora_workspace_bytes(m, k_in, max_rank)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)

    def xa_host(self, rows=None):
        rows = self.m if rows is None else rows
        return from_device_u16(self.xa)[: rows * self.R].reshape(rows, self.R).copy()


def _lora_inputs(seed, m, k_in, n_out, rank, xs, os_, rslora=False):
    rng = W.rng_for(5, salt=seed)
    ad = W.make_adapter(rng, 0, rank, k_in, n_out, 16.0, rslora)
    x = W.bf16_trunc(rng.standard_normal(max(m, 1) * xs).astype(np.float32))
    base = W.bf16_trunc(rng.standard_normal(max(m, 1) * os_).astype(np.float32))
    return ad, x, base


def _check_lora(run, ad, x, xs, base, off, os_, label):
    """xa and the folded region against the oracle; everything else bit-exact."""
    m, k_in, n_out, Rk = run.m, run.k_in, run.n_out, run.R
    w = O.pack_slots([ad], 1, Rk)[0]
    xa_o, out_o = O.lora_delta(w, k_in, n_out, Rk, x, xs, m, base, off, os_)
    X = x[np.arange(m)[:, None] * xs + np.arange(k_in)]
    assert_xa_close(run.xa_host(), xa_o, f"{label} xa", abs_sums_rows(X, w.A),
                    shrink_depth("bgmv", k_in, Rk))
    out_g = run.base.body()
    rows_o = off + np.arange(m)[:, None] * os_ + np.arange(n_out)
    xa64 = O.bf16_to_f64(xa_o)
    delta = O.round_bf16(xa64 @ w.b64().T)
    sabs = np.abs(xa64) @ np.abs(w.b64()).T
    assert_out_close(out_g[rows_o], out_o[rows_o], f"{label} out", delta=delta,
                     scale=float(w.scale), sabs_d=sabs, depth_d=expand_depth("bgmv", Rk))
    outside = np.ones(out_g.size, bool)
    outside[rows_o.ravel()] = False
    assert np.array_equal(out_g[outside], base[outside]), f"{label}: outside [0, n_out) changed"


@pytest.mark.parametrize("m,k_in,n_out,max_rank,rank", [
    (1, 4096, 4096, 16, 8),        # the pages' m == 1 GEMV pair
    (2, 256, 264, 8, 8),
    (48, 1000, 520, 24, 20),       # up to the pages' row-loop threshold
    (49, 2056, 264, 32, 32),       # just past it: their GEMM path
    (130, 512, 768, 128, 100),     # rank 128, ragged tiles
    (1000, 12288, 1032, 64, 64),   # k split over 24 chunks
    (4096, 4096, 4096, 16, 16),    # a prefill-sized batch
], ids=lambda v: str(v))
def test_lora_delta_shapes(m, k_in, n_out, max_rank, rank):
    dev = require_gpu()
    say(f"case: unrouted m={m} k_in={k_in} n_out={n_out} r={max_rank}")
    ad, x, base = _lora_inputs(m % 97, m, k_in, n_out, rank, k_in, n_out, rslora=m % 2 == 1)
    run = LoraRun(ad, m, k_in, n_out, max_rank, x, base, dev)
    R.check(R.rld_lora_delta(run.sp.pair, run.x.ptr(), k_in, m, run.base.ptr(), n_out, run.xa,
                             run.ws, run.ws_bytes), "rld_lora_delta")
    torch.cuda.synchronize()
    _check_lora(run, ad, x, k_in, base, 0, n_out, f"unrouted m={m}")


def test_lora_delta_strided_two_stage():
    """Padded x rows, the output region inside wider rows (as the K region of a
    [Q|K|V] row), through the separate shrink and expand entry points."""
    dev = require_gpu()
    m, k_in, n_out, Rk = 77, 1536, 264, 32
    xs, os_, off = k_in + 8, 3 * n_out, n_out
    say("case: unrouted strided")
    ad, x, base = _lora_inputs(3, m, k_in, n_out, 24, xs, os_)
    run = LoraRun(ad, m, k_in, n_out, Rk, x, base, dev)
    R.check(R.rld_lora_shrink(run.sp.pair, run.x.ptr(), xs, m, run.xa, run.ws, run.ws_bytes),
            "rld_lora_shrink")
    R.check(R.rld_lora_expand_fold(run.sp.pair, run.xa, m, run.base.ptr(off), os_),
            "rld_lora_expand_fold")
    torch.cuda.synchronize()
    _check_lora(run, ad, x, xs, base, off, os_, "unrouted strided")


def test_lora_delta_equals_routed_and_single_rows():
    """The pages: the routed fold is byte-identical to row-by-row unrouted calls.
    Here m rows of rld_lora_delta == m one-row rld_lora_delta calls == rld_bgmv
    with every row on the slot holding the same pair, bit for bit (xa and out),
    with and without a k split."""
    dev = require_gpu()
    for m, k_in, n_out, Rk in ((150, 12288, 520, 64), (70, 512, 1032, 16)):
        say(f"case: unrouted vs routed vs single rows k_in={k_in}")
        ad, x, base = _lora_inputs(7, m, k_in, n_out, Rk, k_in, n_out)
        full = LoraRun(ad, m, k_in, n_out, Rk, x, base, dev)
        R.check(R.rld_lora_delta(full.sp.pair, full.x.ptr(), k_in, m, full.base.ptr(), n_out,
                                 full.xa, full.ws, full.ws_bytes), "rld_lora_delta")
        torch.cuda.synchronize()
        xa_full, out_full = full.xa_host(), full.base.body()
        rows = LoraRun(ad, m, k_in, n_out, Rk, x, base, dev)
        xa1s = []
        for i in range(m):
            R.check(R.rld_lora_delta(rows.sp.pair, rows.x.ptr(i * k_in), k_in, 1,
                                     rows.base.ptr(i * n_out), n_out, rows.xa, rows.ws,
                                     rows.ws_bytes), "one-row rld_lora_delta")
            torch.cuda.synchronize()
            xa1s.append(rows.xa_host(1)[0])
        assert np.array_equal(np.stack(xa1s), xa_full)
        assert np.array_equal(rows.base.body(), out_full)
        routed = LoraRun(ad, m, k_in, n_out, Rk, x, base, dev)
        seq = dev_i32(np.zeros(m, np.int32), dev)
        wsb = R.rld_bgmv_workspace_bytes(m, k_in, Rk, 1)
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
        R.check(R.rld_bgmv(routed.sp.route.route, routed.x.ptr(), k_in, seq, m,
                           routed.base.ptr(), n_out, routed.xa, ws, wsb), "rld_bgmv")
        torch.cuda.synchronize()
        assert np.array_equal(routed.xa_host(), xa_full)
        assert np.array_equal(routed.base.body(), out_full)


# ------------------------------------------------------------ graph safety ---

def test_bgmv_graph_new_routing_each_replay():
    """The graph-safe contract: rld_bgmv is captured once, and before every
    replay new seq_slot contents (including out-of-range slots) are written into
    the same device buffer.  Each replay meets the oracle for its own routing."""
    dev = require_gpu()
    wl = W.bgmv_custom(31, 96, 4096, 1032, 16, 8, (8, 16), base_frac=0.1)
    say("case: bgmv graph, new seq_slot per replay")
    run = BgmvRun(wl, dev)
    pristine = run.bufs["out"].t.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run.run_call(0, stream=s)
    rng = np.random.default_rng(77)
    for rep in range(4):
        seq = rng.integers(-2, 10, size=wl.n).astype(np.int32)  # 8, 9: beyond max_loras
        run.seq.copy_(torch.from_numpy(seq))
        run.bufs["out"].t.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        run.wl = dataclasses.replace(wl, seq_slot=seq)
        run.xa_by_call = [from_device_u16(run.xa)[: wl.n * 16].reshape(wl.n, 16).copy()]
        compare_bgmv(run, f"replay {rep}")
        _base_rows_xa_zero(run.wl, run)


def test_bgmv_multi_graph_new_routing_each_replay():
    """rld_bgmv_multi (q, k and v of the attention decode) captured once;
    before every replay new seq_slot contents (out-of-range slots included) go
    into the captured buffer, and each replay is bit-identical, xa and outputs,
    to one eager rld_bgmv per route on that routing."""
    dev = require_gpu()
    wl = W.bgmv_attn_decode()
    idx = [i for i, c in enumerate(wl.calls) if c.module in ("q", "k", "v")]
    cs = [wl.calls[i] for i in idx]
    say("case: bgmv multi graph, new seq_slot per replay")
    run = BgmvRun(wl, dev)
    pristine = {k: b.t.clone() for k, b in run.bufs.items()}
    xas = [torch.zeros(wl.n * 16 + 8, dtype=torch.int16, device=dev) for _ in cs]
    wsb = R.rld_bgmv_multi_workspace_bytes(wl.n, cs[0].k_in, 16, len(cs))
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    args = ([run.routes[i].route for i in idx], run.bufs[cs[0].x_buf].ptr(), cs[0].x_row_stride,
            run.seq, wl.n, [run.bufs[c.out_buf].ptr(c.out_offset) for c in cs],
            [c.out_row_stride for c in cs], xas, ws, wsb)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        R.check(R.rld_bgmv_multi(*args, stream=s), "rld_bgmv_multi (capture)")
    rng = np.random.default_rng(78)
    for rep in range(3):
        seq = rng.integers(-2, 18, size=wl.n).astype(np.int32)  # 16, 17: beyond max_loras
        run.seq.copy_(torch.from_numpy(seq))
        for k, b in run.bufs.items():
            b.t.copy_(pristine[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = BgmvRun(dataclasses.replace(wl, seq_slot=seq), dev)
        for i, xa in zip(idx, xas):
            ref.run_call(i)
            torch.cuda.synchronize()
            want = from_device_u16(ref.xa)[: wl.n * 16]
            assert np.array_equal(from_device_u16(xa)[: wl.n * 16], want), \
                f"replay {rep}: xa of {wl.calls[i].module}"
        got, exp = run.outputs(), ref.outputs()
        for k in got:
            assert np.array_equal(got[k], exp[k]), f"replay {rep}: buffer {k}"


def test_grouped_graph_new_routing_each_replay():
    """The same for the grouped fold: every window of a projection (k split)
    captured once; before every replay the device expert_offsets,
    sorted_token_ids and row_adapter buffers get the routing of a different
    batch of the same size.  Each replay meets the oracle for its routing."""
    dev = require_gpu()
    wl = _small_grouped(projections=("gate",), hidden=2056)
    p = wl.projections[0]
    say("case: grouped graph, new routing per replay")
    run = GroupedRun(wl, p, dev)
    pristine = run.base.t.clone()
    wins = grouped_windows(wl.te, wl.cap)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for lo, hi in wins:
            R.check(R.rld_moe_grouped(run.route.route, run.x, p.k_in, p.x_gather, wl.num_tokens,
                                      run.off, wl.num_experts, run.stid, run.rad, lo, hi,
                                      run.base.ptr(), p.n_out, run.xa, run.cap, run.ws,
                                      run.ws_bytes, s), "captured rld_moe_grouped")
    for rep, seed in enumerate((41, 42, 43)):
        other = _small_grouped(seed=seed, projections=("gate",), hidden=2056)
        assert other.te == wl.te and other.num_experts == wl.num_experts
        run.off.copy_(torch.from_numpy(other.expert_offsets.astype(np.int32)))
        run.stid.copy_(torch.from_numpy(other.sorted_token_ids.astype(np.int32)))
        run.rad.copy_(torch.from_numpy(other.row_adapter.astype(np.int32)))
        run.base.t.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the new routing over this workload's adapters, x and base rows
        wl2 = W.MoeGroupedWorkload(**{**wl.__dict__, "expert_offsets": other.expert_offsets,
                                      "sorted_token_ids": other.sorted_token_ids,
                                      "row_adapter": other.row_adapter,
                                      "sorted_expert": other.sorted_expert})
        base = p.base.ravel().copy()
        for lo, hi in wins:
            _, base = oracle_grouped_window(wl2, p, lo, hi, base)
        assert_out_close(run.base.body(), base, f"grouped replay {rep}")
