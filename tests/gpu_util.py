"""Shared helpers of the GPU tests: device runs through the C ABI, comparisons
against the oracle at the stated tolerances."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
import routed_lora_delta_amd as R
from routed_lora_delta_amd.pool import (DenseRoute, MoeRoute, from_device_u16, grouped_windows,
                                        to_device_u16)

CANARY = 0x7E5A  # a finite BF16 pattern the fold never writes into guard bands
GUARD = 512      # guard elements before and after every output buffer


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# Every comparison against the oracle appends one record here; tests/conftest.py
# writes them out at the end of the session (RLD_PARITY_OUT), so the number of
# elements that needed the widened rules below is published rather than dropped.
PARITY_RECORDS = []


def _record(kind, label, size, exact, within, widened):
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    PARITY_RECORDS.append(dict(test=test, label=label, kind=kind, elements=int(size),
                               bit_exact=int(exact), within_stated=int(within),
                               widened=int(widened)))


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def dev_i32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)


class Guarded:
    """A device BF16 buffer with canary guard bands on both sides."""

    def __init__(self, host_bits: np.ndarray, device):
        full = np.full(host_bits.size + 2 * GUARD, CANARY, np.uint16)
        full[GUARD:GUARD + host_bits.size] = host_bits.ravel()
        self.t = to_device_u16(full, device)
        self.size = host_bits.size

    def ptr(self, elem_offset=0) -> int:
        return self.t.data_ptr() + 2 * (GUARD + elem_offset)

    def body(self) -> np.ndarray:
        full = from_device_u16(self.t)
        assert np.all(full[:GUARD] == CANARY), "guard band before the buffer was written"
        assert np.all(full[GUARD + self.size:] == CANARY), "guard band after the buffer was written"
        return full[GUARD:GUARD + self.size]


# --------------------------------------------------------------- tolerances --

def ordered(bits):
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def ulp_diff(a, b):
    return np.abs(ordered(a) - ordered(b))


def shrink_depth(path: str, k_in: int, max_rank: int) -> int:
    """Longest chain of fp32 roundings a contraction result passes through in
    the kernels (an upper bound): 32 for one MFMA's internal 32-term sum, plus
    the sequential K steps, plus the fixed-order reductions after them."""
    if path == "bgmv":
        kc = min(256 if max_rank <= 16 else 512, k_in)
        nch = -(-k_in // kc)
        steps = -(-kc // 32)
        return 32 + -(-steps // 4) + 4 + nch
    if path == "grouped":
        if 1024 < k_in <= 2048 and max_rank <= 32:
            return 32 + 4 + 16 + 1  # one chunk over sixteen waves of four steps
        kc = 512 if k_in > 1024 else (512 if k_in <= 512 else (768 if k_in <= 768 else 1024))
        return 32 + kc // 128 + 4 + -(-k_in // kc)
    if path == "gather":
        return 8 * -(-k_in // 512) + 6
    raise ValueError(path)


def expand_depth(path: str, max_rank: int) -> int:
    return max_rank if path == "gather" else 32 + -(-max_rank // 32)


def assert_xa_close(gpu, ora, label="", s_abs=None, depth=None, max_frac=1e-3):
    """xa (or delta) within 1 BF16 ulp of the oracle.

    The oracle's contraction is exact; the GPU sums in fp32.  Where the result
    is close to zero after cancellation, the fp32 summation error can exceed
    one BF16 ulp of the result.  An element that misses the 1-ulp rule is
    accepted only if its error is inside the rigorous fp32 summation bound
    gamma_D * sum|terms| (gamma_D = D u / (1 - D u), u = 2^-24, D the kernel's
    summation depth) plus one ulp, and such elements stay below max_frac of
    the total.  s_abs may be a callable that returns the sums.  Returns
    (elements off by one ulp, elements under the bound)."""
    gpu = np.asarray(gpu, np.uint16)
    ora = np.asarray(ora, np.uint16)
    d = ulp_diff(gpu, ora)
    bad = d > 1
    nb = int(np.count_nonzero(bad))
    if nb:
        assert s_abs is not None and depth is not None, (
            f"{label}: {nb} elements differ by more than 1 ulp, first "
            f"{np.argwhere(bad)[:5].tolist()}")
        if callable(s_abs):  # computed only when an element needs it
            s_abs = s_abs()
        u = 2.0 ** -24
        gamma = depth * u / (1 - depth * u)
        g64, o64 = O.bf16_to_f64(gpu), O.bf16_to_f64(ora)
        ulp = np.abs(O.bf16_to_f64(ora ^ 1) - o64)  # spacing at the oracle value
        allowed = gamma * np.broadcast_to(s_abs, gpu.shape) + ulp
        over = bad & (np.abs(g64 - o64) > allowed)
        assert not np.any(over), (f"{label}: {int(np.count_nonzero(over))} elements outside the "
                                  f"fp32 summation bound, first {np.argwhere(over)[:5].tolist()}")
        assert nb <= max(1, max_frac * gpu.size), f"{label}: {nb} elements beyond 1 ulp"
    n1 = int(np.count_nonzero(d == 1))
    _record("xa", label, gpu.size, np.count_nonzero(d == 0), n1, nb)
    return n1, nb


def _spacing(bits):
    """BF16 spacing at each value (distance to the neighbour away from zero)."""
    b = np.asarray(bits, np.uint16)
    v = np.abs(O.bf16_to_f64(b))
    nxt = np.abs(O.bf16_to_f64((b & 0x7FFF) + 1))
    return np.abs(nxt - v)


def assert_out_close(gpu, ora, label="", delta=None, scale=None, sabs_d=None, depth_d=None,
                     max_frac=1e-4):
    """Folded output within 2 BF16 ulp or 1e-3 absolute of the oracle.

    The delta itself may differ from the oracle's by one BF16 ulp (or, near
    zero, by the fp32 summation bound); the fold multiplies that difference by
    the slot's scale.  An output outside the stated rule is accepted only if
    |gpu - oracle| <= |scale| * (2 spacing(delta) + gamma_D sum|xa*B|) + 2
    spacing(out), i.e. exactly what an allowed delta difference produces
    through out = bf16(base + scale * delta), and such outputs stay below
    max_frac of the total.  Returns (outputs that differ, outputs accepted by
    the derived bound)."""
    gpu = np.asarray(gpu, np.uint16)
    ora = np.asarray(ora, np.uint16)
    d = ulp_diff(gpu, ora)
    absd = np.abs(O.bf16_to_f64(gpu) - O.bf16_to_f64(ora))
    bad = (d > 2) & ~(absd <= 1e-3)
    nb = int(np.count_nonzero(bad))
    if nb:
        assert delta is not None and scale is not None, (
            f"{label}: {nb} outputs outside tolerance, first {np.argwhere(bad)[:5].tolist()}")
        u = 2.0 ** -24
        extra = 0.0
        if sabs_d is not None:
            extra = depth_d * u / (1 - depth_d * u) * sabs_d
        allowed = np.abs(scale) * (2 * _spacing(delta) + extra) + 2 * _spacing(ora)
        over = bad & (absd > allowed)
        assert not np.any(over), (f"{label}: {int(np.count_nonzero(over))} outputs outside the "
                                  f"derived fold bound, first {np.argwhere(over)[:5].tolist()}")
        assert nb <= max(1, max_frac * gpu.size), f"{label}: {nb} outputs beyond 2 ulp / 1e-3"
    nd = int(np.count_nonzero(d))
    _record("out", label, gpu.size, gpu.size - nd, nd - nb, nb)
    return nd, nb


# ------------------------------------------------------------------- BGMV ----

class BgmvRun:
    """Device state of one BgmvWorkload: routes, guarded buffers, scratch."""

    def __init__(self, wl, device):
        self.wl = wl
        self.device = device
        self.seq = dev_i32(wl.seq_slot, device)
        self.bufs = {k: Guarded(v, device) for k, v in wl.buffers.items()}
        self.routes = [DenseRoute(c.adapters, c.max_loras, c.max_rank, c.k_in, c.n_out, device)
                       for c in wl.calls]
        rmax = max(c.max_rank for c in wl.calls)
        self.xa = torch.zeros(max(1, wl.n) * rmax + 8, dtype=torch.int16, device=device)
        ws = max(R.rld_bgmv_workspace_bytes(wl.n, c.k_in, c.max_rank, c.max_loras)
                 for c in wl.calls)
        self.ws_bytes = ws
        self.ws = torch.zeros(max(ws, 16) // 4 + 4, dtype=torch.float32, device=device)
        self.xa_by_call = []

    def run_call(self, i, stream=None):
        c = self.wl.calls[i]
        st = R.rld_bgmv(self.routes[i].route, self.bufs[c.x_buf].ptr(), c.x_row_stride, self.seq,
                        self.wl.n, self.bufs[c.out_buf].ptr(c.out_offset), c.out_row_stride,
                        self.xa, self.ws, self.ws_bytes, stream)
        R.check(st, f"rld_bgmv {c.module}")

    def run_call_two_stage(self, i, stream=None):
        """The same call through rld_bgmv_shrink then rld_bgmv_expand_fold."""
        c = self.wl.calls[i]
        R.check(R.rld_bgmv_shrink(self.routes[i].route, self.bufs[c.x_buf].ptr(), c.x_row_stride,
                                  self.seq, self.wl.n, self.xa, self.ws, self.ws_bytes, stream),
                f"rld_bgmv_shrink {c.module}")
        R.check(R.rld_bgmv_expand_fold(self.routes[i].route, self.xa, self.seq, self.wl.n,
                                       self.bufs[c.out_buf].ptr(c.out_offset), c.out_row_stride,
                                       stream), f"rld_bgmv_expand_fold {c.module}")

    def run_multi(self, idx, stream=None):
        """Calls idx (same input buffer and stride) in one rld_bgmv_multi; returns
        each route's xa [n, max_rank]."""
        cs = [self.wl.calls[i] for i in idx]
        assert len({(c.x_buf, c.x_row_stride, c.k_in, c.max_rank) for c in cs}) == 1
        c0 = cs[0]
        xas = [torch.zeros(max(1, self.wl.n) * c0.max_rank + 8, dtype=torch.int16,
                           device=self.device) for _ in cs]
        wsb = R.rld_bgmv_multi_workspace_bytes(self.wl.n, c0.k_in, c0.max_rank, len(cs))
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=self.device)
        st = R.rld_bgmv_multi([self.routes[i].route for i in idx], self.bufs[c0.x_buf].ptr(),
                              c0.x_row_stride, self.seq, self.wl.n,
                              [self.bufs[c.out_buf].ptr(c.out_offset) for c in cs],
                              [c.out_row_stride for c in cs], xas, ws, wsb, stream)
        R.check(st, "rld_bgmv_multi")
        torch.cuda.synchronize()
        return [from_device_u16(x)[: self.wl.n * c0.max_rank].reshape(self.wl.n, c0.max_rank)
                for x in xas]

    def run_all(self, keep_xa=True, two_stage=False):
        self.xa_by_call = []
        for i, c in enumerate(self.wl.calls):
            if two_stage:
                self.run_call_two_stage(i)
            else:
                self.run_call(i)
            if keep_xa:
                torch.cuda.synchronize()
                self.xa_by_call.append(
                    from_device_u16(self.xa)[: self.wl.n * c.max_rank].reshape(self.wl.n, c.max_rank).copy())
        torch.cuda.synchronize()

    def outputs(self):
        return {k: b.body() for k, b in self.bufs.items()}


def abs_sums_bgmv(wl, c):
    """sum_c |x[i,c] * A_s[k,c]| per (row, xa column), for the error bound."""
    out = np.zeros((wl.n, c.max_rank))
    x = wl.buffers[c.x_buf]
    amap = {a.slot: a for a in c.adapters}
    for i in range(wl.n):
        a = amap.get(int(wl.seq_slot[i]))
        if a is None:
            continue
        xi = np.abs(O.bf16_to_f64(x[i * c.x_row_stride: i * c.x_row_stride + c.k_in]))
        out[i, :a.rank] = np.abs(O.bf16_to_f64(a.A)) @ xi
    return out


def abs_sums_rows(xrows_bits, A_bits):
    """sum_c |x[c] * A[k,c]| for one A and a set of x rows."""
    return np.abs(O.bf16_to_f64(xrows_bits)) @ np.abs(O.bf16_to_f64(A_bits)).T


def oracle_bgmv(wl):
    """Oracle over every call of a BgmvWorkload, in call order; returns (xa per
    call, final buffers)."""
    bufs = {k: v.copy() for k, v in wl.buffers.items()}
    xas = []
    for c in wl.calls:
        slots = O.pack_slots(c.adapters, c.max_loras, c.max_rank)
        xa, out = O.bgmv(slots, c.k_in, c.n_out, c.max_rank, bufs[c.x_buf], c.x_row_stride,
                         wl.seq_slot, wl.n, bufs[c.out_buf], c.out_offset, c.out_row_stride)
        bufs[c.out_buf] = out
        xas.append(xa)
    return xas, bufs


def oracle_delta_bgmv(wl, c, xa_o):
    """Per output element of one call: the oracle's delta (from the oracle's
    xa), the slot scale and sum|xa*B|, laid out like the call's output buffer
    (zeros elsewhere)."""
    size = wl.buffers[c.out_buf].size
    dl = np.zeros(size, np.uint16)
    sc = np.zeros(size)
    sab = np.zeros(size)
    slots = O.pack_slots(c.adapters, c.max_loras, c.max_rank)
    for i in range(wl.n):
        s = int(wl.seq_slot[i])
        if not (0 <= s < c.max_loras) or slots[s] is None:
            continue
        o0 = c.out_offset + i * c.out_row_stride
        xa64 = O.bf16_to_f64(xa_o[i])
        dl[o0:o0 + c.n_out] = O.round_bf16(slots[s].b64() @ xa64)
        sc[o0:o0 + c.n_out] = float(slots[s].scale)
        sab[o0:o0 + c.n_out] = np.abs(slots[s].b64()) @ np.abs(xa64)
    return dl, sc, sab


def compare_bgmv(run: BgmvRun, label: str):
    xas, bufs = oracle_bgmv(run.wl)
    outs = run.outputs()
    stats = {}
    for i, c in enumerate(run.wl.calls):
        stats[c.module + ".xa"] = assert_xa_close(
            run.xa_by_call[i], xas[i], f"{label}/{c.module} xa",
            s_abs=abs_sums_bgmv(run.wl, c), depth=shrink_depth("bgmv", c.k_in, c.max_rank))
    stats.update(compare_bgmv_outputs(run.wl, outs, label, (xas, bufs)))
    return stats


def compare_bgmv_outputs(wl, outs, label, oracle=None):
    """Every buffer of a BgmvWorkload after all its calls (outs: name -> BF16
    bits) against the oracle: folded regions within the output tolerance,
    everything else (base rows, strided gaps, inputs) bit-exact."""
    xas, bufs = oracle if oracle is not None else oracle_bgmv(wl)
    stats = {}
    out_bufs = {c.out_buf for c in wl.calls}
    for k in bufs:
        if k in out_bufs:
            size = bufs[k].size
            dl, sc, sab = np.zeros(size, np.uint16), np.zeros(size), np.zeros(size)
            for i, c in enumerate(wl.calls):
                if c.out_buf == k:
                    d1, s1, a1 = oracle_delta_bgmv(wl, c, xas[i])
                    m = s1 != 0
                    dl[m], sc[m], sab[m] = d1[m], s1[m], a1[m]
            depth = max(expand_depth("bgmv", c.max_rank) for c in wl.calls)
            stats[k + ".out"] = assert_out_close(outs[k], bufs[k], f"{label}/{k}", dl, sc, sab,
                                                 depth)
        else:
            assert np.array_equal(outs[k], bufs[k]), f"{label}: input buffer {k} changed"
        # base rows and everything outside the folded regions: bit-exact
        touched = np.zeros(bufs[k].size, bool)
        for c in wl.calls:
            if c.out_buf != k:
                continue
            for r in range(wl.n):
                s = int(wl.seq_slot[r])
                if 0 <= s < c.max_loras and any(a.slot == s for a in c.adapters):
                    o0 = c.out_offset + r * c.out_row_stride
                    touched[o0:o0 + c.n_out] = True
        assert np.array_equal(outs[k][~touched], wl.buffers[k][~touched]), (
            f"{label}: {k} changed outside the folded rows/regions")
    return stats


# -------------------------------------------------------------------- MoE ----

def run_gather(wl, device, row_adapter="wl", separate=False):
    """The gather fold through rld_moe_gather (one launch), or with
    separate=True through rld_moe_gather_shrink then _expand_fold."""
    ra = wl.row_adapter if row_adapter == "wl" else row_adapter
    route = MoeRoute(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank, wl.k_in, wl.n_out,
                     device)
    x = to_device_u16(wl.x.ravel(), device)
    base = Guarded(wl.base.ravel(), device)
    idx = dev_i32(wl.indices, device)
    rad = dev_i32(ra, device) if ra is not None else None
    xa = torch.zeros(wl.n_rows * wl.max_rank + 8, dtype=torch.int16, device=device)
    if separate:
        R.check(R.rld_moe_gather_shrink(route.route, x, wl.k_in, idx, rad, wl.top_k, wl.n_rows,
                                        xa), "rld_moe_gather_shrink")
        R.check(R.rld_moe_gather_expand_fold(route.route, xa, idx, rad, wl.top_k, wl.n_rows,
                                             base.ptr(), wl.n_out), "rld_moe_gather_expand_fold")
    else:
        R.check(R.rld_moe_gather(route.route, x, wl.k_in, idx, rad, wl.top_k, wl.n_rows,
                                 base.ptr(), wl.n_out, xa), "rld_moe_gather")
    torch.cuda.synchronize()
    return (from_device_u16(xa)[: wl.n_rows * wl.max_rank].reshape(wl.n_rows, wl.max_rank),
            base.body())


def abs_sums_gather(wl, row_adapter="wl"):
    ra = wl.row_adapter if row_adapter == "wl" else row_adapter
    pairs = {(a.slot, a.expert): a for a in wl.adapters}
    out = np.zeros((wl.n_rows, wl.max_rank))
    for rho in range(wl.n_rows):
        s = int(ra[rho // wl.top_k]) if ra is not None else 0
        a = pairs.get((s, int(wl.indices[rho])))
        if a is not None:
            out[rho, :a.rank] = abs_sums_rows(wl.x[rho][None], a.A)[0]
    return out


def abs_sums_grouped(wl, p, lo, hi, row_adapter="wl", stid=None):
    ra = wl.row_adapter if row_adapter == "wl" else row_adapter
    stid = wl.sorted_token_ids if stid is None else stid
    pairs = {(a.slot, a.expert): a for a in p.adapters}
    out = np.zeros((hi - lo, wl.max_rank))
    for r in range(lo, hi):
        t = int(stid[r])
        if not 0 <= t < wl.num_tokens:
            continue
        s = int(ra[t]) if ra is not None else 0
        a = pairs.get((s, int(wl.sorted_expert[r])))
        if a is not None:
            xr = p.x[t] if p.x_gather else p.x[r]
            out[r - lo, :a.rank] = abs_sums_rows(xr[None], a.A)[0]
    return out


def oracle_gather(wl, row_adapter="wl"):
    ra = wl.row_adapter if row_adapter == "wl" else row_adapter
    pairs = O.pack_expert_pairs(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank)
    return O.moe_gather(pairs, wl.num_experts, wl.k_in, wl.n_out, wl.max_rank, wl.x.ravel(),
                        wl.k_in, wl.indices, ra, wl.top_k, wl.n_rows, wl.base.ravel(), wl.n_out)


class GroupedRun:
    """Device state of one grouped projection.  stid: "wl" (the workload's
    sorted_token_ids), an int32 array that replaces it, or None (a NULL
    pointer).  table_experts: build the route's tables for experts
    [0, table_experts) only, while the offsets still list wl.num_experts."""

    def __init__(self, wl, proj, device, cap=None, row_adapter="wl", stid="wl",
                 table_experts=None):
        self.wl, self.p, self.device = wl, proj, device
        self.cap = cap or wl.cap
        self.ra = wl.row_adapter if row_adapter == "wl" else row_adapter
        te_ = table_experts or wl.num_experts
        ads = [a for a in proj.adapters if a.expert < te_]
        self.route = MoeRoute(ads, wl.max_loras, te_, wl.max_rank, proj.k_in, proj.n_out, device)
        self.x = to_device_u16(proj.x.ravel(), device)
        self.base = Guarded(proj.base.ravel(), device)
        self.off = dev_i32(wl.expert_offsets, device)
        st = wl.sorted_token_ids if isinstance(stid, str) else stid
        self.stid = dev_i32(st, device) if st is not None else None
        self.rad = dev_i32(self.ra, device) if self.ra is not None else None
        self.xa = torch.zeros(self.cap * wl.max_rank + 8, dtype=torch.int16, device=device)
        self.ws_bytes = R.rld_moe_grouped_workspace_bytes(self.cap, proj.k_in, wl.max_rank,
                                                          wl.max_loras, wl.num_experts)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)

    def run(self, windows=None, keep_xa=True, separate=False):
        """Every window through rld_moe_grouped (which may fuse the two
        stages), or with separate=True through rld_moe_grouped_shrink then
        rld_moe_grouped_expand_fold."""
        wl, p = self.wl, self.p
        windows = windows if windows is not None else grouped_windows(wl.te, self.cap)
        xas = []
        for lo, hi in windows:
            if separate:
                R.check(R.rld_moe_grouped_shrink(self.route.route, self.x, p.k_in, p.x_gather,
                                                 wl.num_tokens, self.off, wl.num_experts,
                                                 self.stid, self.rad, lo, hi, self.xa, self.cap,
                                                 self.ws, self.ws_bytes),
                        "rld_moe_grouped_shrink")
                R.check(R.rld_moe_grouped_expand_fold(self.route.route, self.xa, wl.num_tokens,
                                                      self.off, wl.num_experts, self.stid,
                                                      self.rad, lo, hi, self.base.ptr(),
                                                      p.n_out),
                        "rld_moe_grouped_expand_fold")
            else:
                R.check(R.rld_moe_grouped(self.route.route, self.x, p.k_in, p.x_gather,
                                          wl.num_tokens, self.off, wl.num_experts, self.stid,
                                          self.rad, lo, hi, self.base.ptr(), p.n_out, self.xa,
                                          self.cap, self.ws, self.ws_bytes),
                        "rld_moe_grouped")
            if keep_xa:
                torch.cuda.synchronize()
                xas.append(from_device_u16(self.xa)[: (hi - lo) * wl.max_rank]
                           .reshape(hi - lo, wl.max_rank).copy())
        torch.cuda.synchronize()
        return xas


def oracle_grouped_window(wl, p, lo, hi, base, row_adapter="wl", stid="wl", table_experts=None):
    ra = wl.row_adapter if row_adapter == "wl" else row_adapter
    st = wl.sorted_token_ids if isinstance(stid, str) else stid
    te_ = table_experts or wl.num_experts
    ads = [a for a in p.adapters if a.expert < te_]
    pairs = O.pack_expert_pairs(ads, wl.max_loras, te_, wl.max_rank)
    return O.moe_grouped(pairs, te_, p.k_in, p.n_out, wl.max_rank, p.x.ravel(), p.k_in,
                         p.x_gather, wl.num_tokens, wl.expert_offsets, st, ra, lo, hi, base,
                         p.n_out)
