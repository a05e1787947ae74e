"""Throughput of the routed LoRA fold on one MI355X.

One step is one pass of every hot-path call over one batch of seeded synthetic
inputs shaped like the routed-LoRA workloads:
  attention decode BGMV   n=64, hidden 4096, q/k/v/o (k/v inside [Q|K|V] rows)
  FFN decode BGMV         n=256, gate/up 4096->12288, down 12288->4096, 32 slots
  MoE decode gather fold  32 tokens x top-8 of 128 experts, down 768->2048
  MoE grouped prefill     4096 tokens x top-8, te=32768 sorted rows, windows of
                          8192; down 768->2048 and gate/up 2048->768 (x gather)
Every call goes through librld.so's C ABI on torch's current stream.

The step graph keeps a layer's dependencies: the q, k and v folds (and the gate
and up folds, dense or MoE) read the same input and write different outputs,
so they are captured on parallel branches (each with its own xa and
workspace); o follows q/k/v and down follows gate/up.

Timing.  The step is captured once as a HIP graph; timed region A replays it K
times back to back and its wall clock gives ms_per_step and the value.  Timed
regions B and C time every call, one at a time, with HIP events on the launch
stream (their sum is ms_per_step_calls): the
grouped-window calls are issued eagerly, each between two events, right after
a replay of the captured BGMV+gather part (region B), and the BGMV and gather
calls the same way after a replay of the captured grouped part (region C), so
the host is always ahead of the GPU and an event pair brackets exactly one
call.  The kernel with the largest total time is reported against its
roofline: achieved = its algorithmic bytes per launch / its mean launch
duration.  Each workload is also captured alone, its independent calls on
parallel branches as in the step, and timed as that graph after a replay of
the rest of the step (per_workload[*].graph).
Algorithmic bytes are counted from the actual inputs: x rows that fold, A and
B of each distinct (slot[, expert]) pair a call touches, the base rows read
and written, xa written and read, and the index arrays.  A launch that folds
two calls counts both calls' bytes; for the launches that read a shared x
once or keep xa on chip (the MoE gate+up pair launch, the BGMV one-pass form)
the roofline objects also give the rate on the bytes that launch itself must
move (read_once_*).

The CPU oracle (test infrastructure) is timed on a bounded sample of the same
step for the cpu_baseline field only.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed LoRA fold rows/s + achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


# ------------------------------------------------------------- byte counts --

def _bgmv_active(wl, c):
    have = {a.slot for a in c.adapters}
    act = np.array([int(s) in have for s in wl.seq_slot])
    slots = {int(s) for s, a in zip(wl.seq_slot, act) if a}
    return act, slots


def bgmv_bytes(wl, c):
    act, slots = _bgmv_active(wl, c)
    n_act, S, R = int(act.sum()), len(slots), c.max_rank
    idx = 4 * wl.n
    shrink = 2 * (n_act * c.k_in + S * R * c.k_in + wl.n * R) + idx
    expand = 2 * (S * c.n_out * R + n_act * R + 2 * n_act * c.n_out) + idx
    flops = 2 * n_act * R * (c.k_in + c.n_out)
    return shrink, expand, flops, n_act


def bgmv_read_once_bytes(wl, calls, onepass):
    """What one launch serving BGMV calls over the same x rows must itself move:
    the calls' bytes of bgmv_bytes with x read once, over the union of the rows
    any call folds, and, in the one-pass form (which keeps xa on chip), without
    the xa read-back."""
    total, act_any, xa_back = 0, np.zeros(wl.n, bool), 0
    for c in calls:
        sb, eb, _, n_act = bgmv_bytes(wl, c)
        act, _ = _bgmv_active(wl, c)
        total += sb + eb - 2 * n_act * c.k_in
        act_any |= act
        xa_back += 2 * n_act * c.max_rank
    return total + 2 * int(act_any.sum()) * calls[0].k_in - (xa_back if onepass else 0)


def gather_bytes(wl):
    pairs = {(a.slot, a.expert) for a in wl.adapters}
    act, S = 0, set()
    for rho in range(wl.n_rows):
        s = int(wl.row_adapter[rho // wl.top_k]) if wl.row_adapter is not None else 0
        key = (s, int(wl.indices[rho]))
        if key in pairs:
            act += 1
            S.add(key)
    R = wl.max_rank
    idx = 4 * (wl.n_rows + wl.num_tokens)
    shrink = 2 * (act * wl.k_in + len(S) * R * wl.k_in + wl.n_rows * R) + idx
    expand = 2 * (len(S) * wl.n_out * R + act * R + 2 * act * wl.n_out) + idx
    return shrink, expand, 2 * act * R * (wl.k_in + wl.n_out), act


def _grouped_active(wl, p, lo, hi):
    """Sorted rows [lo, hi) that projection p folds: (active mask, token ids,
    slots, experts)."""
    pairs = {(a.slot, a.expert) for a in p.adapters}
    toks = wl.sorted_token_ids[lo:hi]
    exps = wl.sorted_expert[lo:hi]
    slots = (wl.row_adapter[toks] if wl.row_adapter is not None
             else np.zeros(hi - lo, np.int32))
    act = np.array([(int(s), int(e)) in pairs for s, e in zip(slots, exps)], bool)
    return act, toks, slots, exps


def grouped_window_bytes(wl, p, lo, hi):
    act, toks, slots, exps = _grouped_active(wl, p, lo, hi)
    S = len({(int(s), int(e)) for s, e, a in zip(slots, exps, act) if a})
    n_act, R, nw = int(act.sum()), wl.max_rank, hi - lo
    x_rows = len(set(toks[act].tolist())) if p.x_gather else n_act
    idx = 4 * (2 * nw + wl.num_experts + 1)
    shrink = 2 * (x_rows * p.k_in + S * R * p.k_in + nw * R) + idx
    expand = 2 * (S * p.n_out * R + n_act * R + 2 * n_act * p.n_out) + idx
    return shrink, expand, 2 * n_act * R * (p.k_in + p.n_out), n_act


def grouped_pair_read_once_bytes(wl, p, q, lo, hi):
    """What one launch folding projections p and q of window [lo, hi) over the
    same gathered x must itself move: the two calls' bytes of
    grouped_window_bytes with x read once, over the union of the tokens either
    projection folds, and without the xa read-back (the launch writes xa and
    keeps it on chip for the fold)."""
    sb, eb, _, _ = grouped_window_bytes(wl, p, lo, hi)
    sb2, eb2, _, _ = grouped_window_bytes(wl, q, lo, hi)
    ap, toks, _, _ = _grouped_active(wl, p, lo, hi)
    aq, _, _, _ = _grouped_active(wl, q, lo, hi)
    xp, xq = len(set(toks[ap].tolist())), len(set(toks[aq].tolist()))
    xu = len(set(toks[ap | aq].tolist()))
    return (sb + eb + sb2 + eb2 - 2 * p.k_in * (xp + xq - xu)
            - 2 * wl.max_rank * int(ap.sum() + aq.sum()))


# ------------------------------------------------------ counters and profiles --

PROFILES = os.path.join(ROOT, "profiles")


def source_digest():
    """sha256 of the library's kernel sources and header: counter readings
    taken for other sources do not describe the kernels that run."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "routed_lora_delta_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "rld.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _kernel_key(name):
    """'void rld::bgmv_expand_kernel<2>(rld::BgmvArgs)' -> 'bgmv_expand_kernel'."""
    n = name.split("(")[0].split("<")[0]
    return n.split("::")[-1].strip()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    counter summary in profiles/ (calibrated FETCH_SIZE + WRITE_SIZE), or None
    when there is none for this workload and the current kernel sources.  A
    label "a+b" (a call's two launches, as the shrink and its chunk reduce)
    sums the two kernels' figures."""
    import glob
    if "+" in kernel:
        parts = [measured_traffic(k, workload) for k in kernel.split("+")]
        return None if any(p is None for p in parts) else int(sum(parts))
    digest = source_digest()
    for f in sorted(glob.glob(os.path.join(PROFILES, "*counters*.md"))):
        with open(f) as fh:
            txt = fh.read()
        for block in txt.split("```json")[1:]:
            try:
                d = json.loads(block.split("```")[0])
            except ValueError:
                continue
            if (d.get("source_digest") == digest and d.get("workload") == workload
                    and kernel in d.get("kernels", {})):
                return int(d["kernels"][kernel]["traffic_bytes_per_launch"])
    return None


def summarize(dirs, bench_json=None, workload="step"):
    """Markdown summary of rocprofv3 output directories: kernel-trace stats
    (*_kernel_stats.csv) and FETCH_SIZE / WRITE_SIZE counter runs
    (*_counter_collection.csv) calibrated on the COPY_BYTES copy of
    --copy-calibration (the copy dispatch with the largest reading)."""
    import csv
    import glob
    lines = []
    stats = [f for d in dirs for f in glob.glob(os.path.join(d, "**", "*_kernel_stats.csv"),
                                                 recursive=True)]
    for f in stats:
        rows = list(csv.DictReader(open(f)))
        lines.append(f"Kernel trace statistics ({os.path.relpath(f)}):\n")
        lines.append("| kernel | calls | mean us | min us | max us | share |")
        lines.append("|---|---|---|---|---|---|")
        for r in rows:
            lines.append(f"| {r['Name'][:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                         f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                         f"{float(r['Percentage']):.1f}% |")
        lines.append("")
    traces = [f for d in dirs for f in glob.glob(os.path.join(d, "**", "*_kernel_trace.csv"),
                                                  recursive=True)]
    for f in traces:
        # launches that overlapped no other launch, against all of them: the
        # step graph runs independent calls on parallel branches, and a kernel
        # sharing the chip with another takes longer than one running alone
        ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                    for r in csv.DictReader(open(f)))
        alone = {}
        last_end = -1
        for i, (t0, t1, name) in enumerate(ev):
            nxt = ev[i + 1][0] if i + 1 < len(ev) else None
            solo = t0 >= last_end and (nxt is None or nxt >= t1)
            last_end = max(last_end, t1)
            if "rld::" not in name:
                continue
            k = alone.setdefault(_kernel_key(name), [[], []])
            k[0].append((t1 - t0) / 1e3)
            if solo:
                k[1].append((t1 - t0) / 1e3)
        lines.append(f"Launches that ran alone ({os.path.relpath(f)}):\n")
        lines.append("| kernel | launches | alone | mean us, all | mean us, alone |")
        lines.append("|---|---|---|---|---|")
        for k, (al, so) in sorted(alone.items()):
            lines.append(f"| {k} | {len(al)} | {len(so)} | {np.mean(al):.3f} | "
                         f"{(np.mean(so) if so else float('nan')):.3f} |")
        lines.append("")
    counters = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                counters.setdefault(r["Counter_Name"], []).append(r)
    if counters:
        factor = {}
        per = {}
        for cname, rows in counters.items():
            copies = [float(r["Counter_Value"]) for r in rows
                      if "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower()]
            big = max(copies) if copies else 0.0
            factor[cname] = COPY_BYTES / (big * 1024.0) if big > 0 else None
            for r in rows:
                if "rld::" not in r["Kernel_Name"]:
                    continue
                k = per.setdefault(_kernel_key(r["Kernel_Name"]), {})
                k.setdefault(cname, []).append(float(r["Counter_Value"]))
        lines.append(f"Counter calibration: a {COPY_BYTES >> 20} MiB device copy reads as "
                     + ", ".join(f"{c} {COPY_BYTES / 1024 / factor[c]:.1f} KiB (factor "
                                 f"{factor[c]:.4f})" for c in sorted(factor) if factor[c]) + "\n")
        lines.append("| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | "
                     "HBM MB/dispatch (calibrated) |")
        lines.append("|---|---|---|---|---|")
        out = {"source_digest": source_digest(), "workload": workload,
               "copy_bytes": COPY_BYTES, "factors": factor, "kernels": {}}
        for k, v in sorted(per.items()):
            fk = float(np.mean(v.get("FETCH_SIZE", [0.0])))
            wk = float(np.mean(v.get("WRITE_SIZE", [0.0])))
            tb = fk * 1024 * (factor.get("FETCH_SIZE") or 1.0) + \
                wk * 1024 * (factor.get("WRITE_SIZE") or 1.0)
            out["kernels"][k] = {"dispatches": len(v.get("FETCH_SIZE", v.get("WRITE_SIZE", []))),
                                 "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                                 "traffic_bytes_per_launch": int(tb)}
            lines.append(f"| {k} | {out['kernels'][k]['dispatches']} | {fk:.1f} | {wk:.1f} | "
                         f"{tb / 1e6:.2f} |")
        lines.append("")
        lines.append("```json\n" + json.dumps(out, indent=1) + "\n```")
    if bench_json:
        with open(bench_json) as fh:
            b = json.loads(fh.read().strip().splitlines()[-1])
        lines.append("\nBench line of the same build (kernels: mean us per launch):\n")
        lines.append("| kernel | launches/step | mean us | algorithmic MB/launch | GB/s |")
        lines.append("|---|---|---|---|---|")
        for k, v in b.get("kernels", {}).items():
            lines.append(f"| {k} | {v['launches_per_step']} | {v['avg_us']} | "
                         f"{v['algo_bytes_per_launch'] / 1e6:.2f} | {v['gbs']} |")
        lines.append(f"\nms_per_step {b['ms_per_step']}, value {b['value']} {b['unit']}, "
                     f"roofline {json.dumps(b['roofline'])}")
    return "\n".join(lines)


# ------------------------------------------------------------------ GPU side --

# Independent calls of one step and the order of their groups: in a layer, the
# q, k and v folds (and the gate and up folds) read the same input and write
# different outputs, so they run on parallel branches of the step's graph; o
# follows q/k/v, down follows gate/up.  Module -> (group within its workload,
# lane).  Calls of one module keep one lane (its shrink feeds its expand).  The
# windows of a grouped projection write disjoint rows of its output, so with an
# xa arena and a workspace each they are independent too: window k of a module
# on lane `lane * windows + k`.
LANES = {"q": (0, 0), "k": (0, 1), "v": (0, 2), "o": (1, 0),
         "gate": (0, 0), "up": (0, 1), "down": (1, 0)}
MAX_LANES = 3
# workloads whose first group of folds is one rld_bgmv_multi call
MULTI_TAGS = {"attn"}
# A whole decoder layer ("layer<i>" workloads of the multi-layer decode step):
# q/k/v (one rld_bgmv_multi call), then o, then gate and up (one rld_bgmv_multi
# call: three launches instead of six, 1.82 against 2.09 ms for the 36-layer
# step), then down; layers follow each other.  (As two calls on two graph
# branches gate and up cost the step 2.31 ms against 2.16 ms on one stream: at
# n = 64 and rank 16 the branches' cross-queue waits outweigh the overlap.)
LAYER_LANES = {"q": (0, 0), "k": (0, 1), "v": (0, 2), "o": (1, 0),
               "gate": (2, 0), "up": (2, 0), "down": (3, 0)}


def grouped_shrink_kernel(k_in, max_rank):
    """Kernel that rld_moe_grouped_shrink launches: the sixteen-wave one for
    1024 < k_in <= 2048 at max_rank <= 32, the chunked one otherwise."""
    wide = 1024 < k_in <= 2048 and max_rank <= 32
    return "grouped_shrink_wide_kernel" if wide else "grouped_shrink_kernel"


def grouped_fused(k_in, max_rank, n_out):
    """rld_moe_grouped runs the shrink and the fold of a window as one kernel
    when the wide shrink applies and n_out <= 768."""
    return grouped_shrink_kernel(k_in, max_rank) == "grouped_shrink_wide_kernel" and n_out <= 768


def grouped_pair_fused(pa, pb, wl):
    """rld_moe_grouped_pair folds the two projections in one launch (the same
    input rows, both fusable, at most 512 (slot, expert) pairs)."""
    return (pa.x is pb.x and pa.k_in == pb.k_in
            and grouped_fused(pa.k_in, wl.max_rank, pa.n_out)
            and grouped_fused(pb.k_in, wl.max_rank, pb.n_out)
            and wl.max_loras * wl.num_experts <= 512 and wl.num_experts < 511)


class Step:
    """Device state of the whole step and the ordered list of its calls.  Every
    call has a (group, lane): calls of one group on different lanes are
    independent and run on parallel branches of the captured step (each lane
    has its own xa and workspace); groups run in order."""

    def __init__(self, dev, workloads):
        import torch

        import routed_lora_delta_amd as R
        from routed_lora_delta_amd.pool import (DenseRoute, MoeRoute, SinglePair, grouped_windows,
                                                to_device_u16)

        self.R, self.torch = R, torch
        self.calls = []  # (label, kernel name, fn, algorithmic bytes, flops, rows)
        # label -> bytes a fused launch itself moves (inputs shared by its calls
        # read once, no xa read-back), where that differs from the calls' sum
        self.read_once = {}
        self.outputs = {}  # "<workload>.<buffer or projection>" -> device output tensor
        self.sched = []  # (group, lane) of each call
        self.rows = 0
        keep = []
        group0 = 0

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

        def add(call, module, lane=None, group=None, lanes_map=LANES):
            g, ln = lanes_map.get(module, (0, 0))
            self.calls.append(call)
            self.sched.append((group0 + (g if group is None else group),
                               ln if lane is None else lane))

        seqs = {}     # one device seq_slot per host routing array (layers share theirs)
        shared = {}   # the layers' xa arena and workspaces, allocated once
        self.seqs = seqs
        for tag, wl in workloads:
            layer = tag.startswith("layer")
            lmap = LAYER_LANES if layer else LANES
            if tag in ("attn", "ffn", "lora") or layer:
                if id(wl.seq_slot) not in seqs:
                    seqs[id(wl.seq_slot)] = i32(wl.seq_slot)
                seq = seqs[id(wl.seq_slot)]
                bufs = {k: to_device_u16(v, dev) for k, v in wl.buffers.items()}
                rmax = max(c.max_rank for c in wl.calls)
                if tag == "lora":
                    wsb = max(R.rld_lora_workspace_bytes(wl.n, c.k_in, c.max_rank)
                              for c in wl.calls)
                else:
                    wsb = max(R.rld_bgmv_workspace_bytes(wl.n, c.k_in, c.max_rank, c.max_loras)
                              for c in wl.calls)
                key = (wl.n, rmax, wsb)
                if layer and key in shared:
                    lanes = shared[key]
                else:
                    lanes = [(torch.zeros(wl.n * rmax + 8, dtype=torch.int16, device=dev),
                              torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev))
                             for _ in range(MAX_LANES)]
                    if layer:
                        shared[key] = lanes
                keep += [seq, bufs, lanes]
                for k, b in bufs.items():
                    self.outputs[f"{tag}.{k}"] = b
                # the attention's q, k and v folds read the same rows: one
                # rld_bgmv_multi call for them, and in a decoder layer of the
                # multi-layer step one for gate and up as well.  (In the step's
                # FFN workload gate and up stay two calls on parallel branches,
                # which overlap each other's launch gaps and tails: as one call
                # the FFN's cost in the step was 106 us against 94.)
                multi_groups = [0] if tag in MULTI_TAGS else ([0, 2] if layer else [])
                in_multi = []
                for mg in multi_groups:
                    first = [c for c in wl.calls if lmap.get(c.module, (0, 0))[0] == mg]
                    if len({(c.x_buf, c.x_row_stride, c.k_in, c.max_rank) for c in first}) != 1 \
                            or len(first) < 2:
                        continue
                    in_multi += first
                    c0 = first[0]
                    rts = [DenseRoute(c.adapters, c.max_loras, c.max_rank, c.k_in, c.n_out, dev)
                           for c in first]
                    mwsb = R.rld_bgmv_multi_workspace_bytes(wl.n, c0.k_in, c0.max_rank, len(first))
                    mkey = ("multi", wl.n, c0.k_in, c0.max_rank, len(first))
                    if layer and mkey in shared:
                        mws = shared[mkey]
                    else:
                        mws = torch.zeros(max(mwsb, 16), dtype=torch.uint8, device=dev)
                        if layer:
                            shared[mkey] = mws
                    xas = [lanes[i][0] for i in range(len(first))]
                    outs = [bufs[c.out_buf].data_ptr() + 2 * c.out_offset for c in first]
                    keep += [rts, mws]
                    sb = sum(bgmv_bytes(wl, c)[0] + bgmv_bytes(wl, c)[1] for c in first)
                    fl = sum(bgmv_bytes(wl, c)[2] for c in first)

                    def multi(rts=rts, c0=c0, x=bufs[c0.x_buf].data_ptr(), seq=seq, outs=outs,
                              oss=[c.out_row_stride for c in first], xas=xas, mws=mws,
                              mwsb=mwsb, n=wl.n):
                        return R.rld_bgmv_multi([r.route for r in rts], x, c0.x_row_stride, seq,
                                                n, outs, oss, xas, mws, mwsb)
                    label = (ONEPASS if R.rld_bgmv_launches([r.route for r in rts], wl.n) == 1
                             else "bgmv_multi")
                    mlabel = f"{tag}.{'+'.join(c.module for c in first)}.multi"
                    add((mlabel, label, multi, sb, fl, wl.n * len(first)), c0.module, 0,
                        lanes_map=lmap)
                    self.read_once[mlabel] = bgmv_read_once_bytes(wl, first, label == ONEPASS)
                    self.rows += wl.n * len(first)
                for c in wl.calls:
                    if any(c is f for f in in_multi):
                        continue
                    xa, ws = lanes[lmap.get(c.module, (0, 0))[1]]
                    sb, eb, fl, _ = bgmv_bytes(wl, c)
                    x = bufs[c.x_buf].data_ptr()
                    out = bufs[c.out_buf].data_ptr() + 2 * c.out_offset
                    if tag == "lora":
                        sp = SinglePair(c.adapters[0], c.max_rank, c.k_in, c.n_out, dev)
                        keep.append(sp)

                        def shrink(sp=sp, c=c, x=x, xa=xa, ws=ws, wsb=wsb, m=wl.n):
                            return R.rld_lora_shrink(sp.pair, x, c.x_row_stride, m, xa, ws, wsb)

                        def expand(sp=sp, c=c, out=out, xa=xa, m=wl.n):
                            return R.rld_lora_expand_fold(sp.pair, xa, m, out, c.out_row_stride)
                    else:
                        rt = DenseRoute(c.adapters, c.max_loras, c.max_rank, c.k_in, c.n_out, dev)
                        keep.append(rt)
                        if R.rld_bgmv_launches(rt.route, wl.n) == 1:
                            # one launch: rld_bgmv's one-pass form
                            def fold(rt=rt, c=c, x=x, seq=seq, out=out, xa=xa, ws=ws, wsb=wsb,
                                     n=wl.n):
                                return R.rld_bgmv(rt.route, x, c.x_row_stride, seq, n, out,
                                                  c.out_row_stride, xa, ws, wsb)
                            add((f"{tag}.{c.module}.fold", ONEPASS, fold, sb + eb, fl, wl.n),
                                c.module, lanes_map=lmap)
                            self.read_once[f"{tag}.{c.module}.fold"] = bgmv_read_once_bytes(
                                wl, [c], True)
                            self.rows += wl.n
                            continue

                        def shrink(rt=rt, c=c, x=x, seq=seq, xa=xa, ws=ws, wsb=wsb, n=wl.n):
                            return R.rld_bgmv_shrink(rt.route, x, c.x_row_stride, seq, n, xa, ws,
                                                     wsb)

                        def expand(rt=rt, c=c, out=out, seq=seq, xa=xa, n=wl.n):
                            return R.rld_bgmv_expand_fold(rt.route, xa, seq, n, out,
                                                          c.out_row_stride)
                    add((f"{tag}.{c.module}.shrink", BGMV_SHRINK, shrink, sb, fl / 2, wl.n),
                        c.module, lanes_map=lmap)
                    add((f"{tag}.{c.module}.expand", "bgmv_expand_kernel", expand, eb, fl / 2, 0),
                        c.module, lanes_map=lmap)
                    self.rows += wl.n
            elif tag == "gather":
                rt = MoeRoute(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank, wl.k_in,
                              wl.n_out, dev)
                x = to_device_u16(wl.x.ravel(), dev)
                base = to_device_u16(wl.base.ravel(), dev)
                idx = i32(wl.indices)
                rad = i32(wl.row_adapter)
                xa = torch.zeros(wl.n_rows * wl.max_rank + 8, dtype=torch.int16, device=dev)
                keep += [rt, x, base, idx, rad, xa]
                self.outputs["gather.out"] = base
                sb, eb, fl, _ = gather_bytes(wl)

                # one call: shrink and fold of every flat row in one kernel
                def gfold(rt=rt, x=x, base=base, idx=idx, rad=rad, xa=xa, wl=wl):
                    return R.rld_moe_gather(rt.route, x, wl.k_in, idx, rad, wl.top_k, wl.n_rows,
                                            base, wl.n_out, xa)
                add(("gather.down.fold", "gather_fold_kernel", gfold, sb + eb, fl, wl.n_rows),
                    "")
                self.rows += wl.n_rows
            elif tag == "grouped":
                off = i32(wl.expert_offsets)
                stid = i32(wl.sorted_token_ids)
                rad = i32(wl.row_adapter)
                wins = grouped_windows(wl.te, wl.cap)
                # per lane (module lane x window): xa, and a workspace sized for
                # the largest projection
                wsb = max(R.rld_moe_grouped_workspace_bytes(wl.cap, p.k_in, wl.max_rank,
                                                            wl.max_loras, wl.num_experts)
                          for p in wl.projections)
                lanes = [(torch.zeros(wl.cap * wl.max_rank + 8, dtype=torch.int16, device=dev),
                          torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev))
                         for _ in range(len(wins) * (1 + max(LANES.get(p.name, (0, 0))[1]
                                                             for p in wl.projections)))]
                keep += [off, stid, rad, lanes]
                order = {"gate": 0, "up": 1, "down": 2}
                projs = sorted(wl.projections, key=lambda q: order.get(q.name, 3))
                dev_p = {}
                for p in projs:
                    rt = MoeRoute(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank, p.k_in,
                                  p.n_out, dev)
                    x = to_device_u16(p.x.ravel(), dev)
                    base = to_device_u16(p.base.ravel(), dev)
                    keep += [rt, x, base]
                    dev_p[p.name] = (rt, x, base)
                    self.outputs[f"grouped.{p.name}"] = base
                byname = {p.name: p for p in projs}
                paired = ("gate" in byname and "up" in byname
                          and grouped_pair_fused(byname["gate"], byname["up"], wl))
                # Window k's down rows are the rows its gate and up folds wrote
                # (the activation of sorted row r comes from gate and up of row
                # r), so with the pair call each window is one chain on branch k:
                # gate+up, then down, with no barrier across windows.
                wgroup = 0 if paired else None
                for p in projs:
                    rt, x, base = dev_p[p.name]
                    if paired and p.name == "up":
                        continue  # folded with gate, one call per window
                    for k, (lo, hi) in enumerate(wins):
                        lane = LANES.get(p.name, (0, 0))[1] * len(wins) + k
                        xa, ws = lanes[lane]
                        sb, eb, fl, _ = grouped_window_bytes(wl, p, lo, hi)
                        if paired and p.name == "gate":
                            q = byname["up"]
                            rt_b, _, base_b = dev_p["up"]
                            xa_b = lanes[LANES["up"][1] * len(wins) + k][0]
                            sb2, eb2, fl2, _ = grouped_window_bytes(wl, q, lo, hi)

                            def pair(rt=rt, rt_b=rt_b, x=x, base=base, base_b=base_b, p=p, q=q,
                                     lo=lo, hi=hi, off=off, stid=stid, rad=rad, xa=xa, xa_b=xa_b,
                                     wl=wl, ws=ws, wsb=wsb):
                                return R.rld_moe_grouped_pair(
                                    rt.route, rt_b.route, x, p.k_in, p.x_gather, wl.num_tokens,
                                    off, wl.num_experts, stid, rad, lo, hi, base, p.n_out,
                                    base_b, q.n_out, xa, xa_b, wl.cap, ws, wsb)

                            label = f"grouped.gate+up.[{lo},{hi}).fold"
                            add((label, "grouped_fold_pair_kernel", pair, sb + eb + sb2 + eb2,
                                 fl + fl2, 2 * (hi - lo)), p.name, lane, wgroup)
                            self.read_once[label] = grouped_pair_read_once_bytes(wl, p, q, lo, hi)
                            continue

                        def shrink(rt=rt, x=x, p=p, lo=lo, hi=hi, off=off, stid=stid, rad=rad,
                                   xa=xa, wl=wl, ws=ws, wsb=wsb):
                            return R.rld_moe_grouped_shrink(rt.route, x, p.k_in, p.x_gather,
                                                            wl.num_tokens, off, wl.num_experts,
                                                            stid, rad, lo, hi, xa, wl.cap, ws,
                                                            wsb)

                        def expand(rt=rt, base=base, p=p, lo=lo, hi=hi, off=off, stid=stid,
                                   rad=rad, xa=xa, wl=wl):
                            return R.rld_moe_grouped_expand_fold(rt.route, xa, wl.num_tokens, off,
                                                                 wl.num_experts, stid, rad, lo,
                                                                 hi, base, p.n_out)

                        if grouped_fused(p.k_in, wl.max_rank, p.n_out):
                            # one call: shrink and fold of the window in one kernel
                            def fold(rt=rt, x=x, base=base, p=p, lo=lo, hi=hi, off=off,
                                     stid=stid, rad=rad, xa=xa, wl=wl, ws=ws, wsb=wsb):
                                return R.rld_moe_grouped(rt.route, x, p.k_in, p.x_gather,
                                                         wl.num_tokens, off, wl.num_experts,
                                                         stid, rad, lo, hi, base, p.n_out, xa,
                                                         wl.cap, ws, wsb)

                            add((f"grouped.{p.name}.[{lo},{hi}).fold",
                                 "grouped_fold_wide_kernel", fold, sb + eb, fl, hi - lo),
                                p.name, lane, wgroup)
                            continue
                        add((f"grouped.{p.name}.[{lo},{hi}).shrink",
                             grouped_shrink_kernel(p.k_in, wl.max_rank), shrink, sb, fl / 2,
                             hi - lo), p.name, lane, wgroup)
                        add((f"grouped.{p.name}.[{lo},{hi}).expand", "grouped_expand_kernel",
                             expand, eb, fl / 2, 0), p.name, lane, wgroup)
                self.rows += wl.te * len(projs)
            group0 = max((g for g, _ in self.sched), default=-1) + 1
        self._keep = keep
        self.bytes = sum(c[3] for c in self.calls)
        self.flops = sum(c[4] for c in self.calls)

    def capture(self, idx, stream, parallel=True):
        """One HIP graph of the calls idx (in order), captured on `stream`: each
        group forks its lanes onto side streams and joins them before the next
        group starts (parallel=False: every call on `stream`, in order)."""
        torch = self.torch
        nlanes = 1 + max(ln for _, ln in self.sched)
        side = [None] + [torch.cuda.Stream() for _ in range(nlanes - 1)]
        idx = list(idx)
        g = torch.cuda.CUDAGraph()
        if not parallel:
            with torch.cuda.graph(g, stream=stream):
                for i in idx:
                    if self.calls[i][2]() != 0:
                        raise RuntimeError("call failed during capture: " + self.calls[i][0])
            return g
        with torch.cuda.graph(g, stream=stream):
            groups = sorted({self.sched[i][0] for i in idx})
            for grp in groups:
                members = [i for i in idx if self.sched[i][0] == grp]
                lanes = sorted({self.sched[i][1] for i in members})
                for ln in lanes:
                    if ln:
                        side[ln].wait_stream(stream)
                for ln in lanes:
                    with torch.cuda.stream(stream if ln == 0 else side[ln]):
                        for i in members:
                            if self.sched[i][1] == ln and self.calls[i][2]() != 0:
                                raise RuntimeError("call failed during capture: "
                                                   + self.calls[i][0])
                for ln in lanes:
                    if ln:
                        stream.wait_stream(side[ln])
        return g

    def enqueue(self, events=None):
        """Issue every call on the current stream; events[i] is recorded before
        call i and events[-1] after the last call."""
        for i, (label, _, fn, _, _, _) in enumerate(self.calls):
            if events is not None:
                events[i].record()
            st = fn()
            if st != 0:
                raise RuntimeError(f"{label}: {self.R.rld_status_string(st)}")
        if events is not None:
            events[-1].record()


MODEL_LAYERS = 36


def model_workloads(layers=MODEL_LAYERS):
    """The multi-layer decode step: `layers` decoder layers of Qwen3-8B shapes,
    each with its own pools for all seven projections, one batch routing."""
    import workloads as W
    seq = W.decode_routing()
    return [(f"layer{i}", W.decode_layer(i, seq)) for i in range(layers)]


def select_workloads(name):
    import workloads as W
    out = []
    if name in ("step", "attn"):
        out.append(("attn", W.bgmv_attn_decode()))
    if name in ("step", "ffn"):
        out.append(("ffn", W.bgmv_ffn_decode()))
    if name in ("step", "gather"):
        out.append(("gather", W.moe_gather()))
    if name in ("step", "grouped"):
        out.append(("grouped", W.moe_grouped()))
    if name == "lora":
        out.append(("lora", W.lora_prefill()))
    if name == "model":
        out += model_workloads()
    return out


WORKLOAD_NAMES = {
    "step": "routed-fold step: attn-decode BGMV q/k/v/o n=64 h4096 r16 L16 + ffn-decode BGMV "
            "gate/up/down n=256 4096x12288 r64 L32 + MoE gather down 32tok top8 E128 768->2048 "
            "r16 L8 + MoE grouped down/gate/up 4096tok top8 E128 te32768 cap8192 r32 L4",
    "attn": "attn-decode BGMV q/k/v/o n=64 hidden=4096 r16 L16 ([Q|K|V] stride 6144)",
    "ffn": "ffn-decode BGMV gate/up/down n=256 4096x12288 r64 L32",
    "gather": "MoE gather down 32 tokens top8 E128 768->2048 r16 L8",
    "grouped": "MoE grouped down/gate/up 4096 tokens top8 E128 te=32768 cap=8192 r32 L4",
    "lora": "unrouted single adapter, prefill m=4096, FFN gate/up 4096->12288, down "
            "12288->4096, r64",
    "model": f"decode step of {MODEL_LAYERS} Qwen3-8B layers: q/k/v/o and gate/up/down folds "
             "per layer (own pools), n=64, 16 slots r16, one batch routing",
}

# The BGMV shrink entry point is two launches when k_in is split (the shrink,
# then the chunk reduce); the bench times the pair as one entry.
BGMV_SHRINK = "bgmv_shrink_kernel+bgmv_reduce_kernel"
# launches behind one bench entry (the step's BGMV calls all split k_in)
ONEPASS = "bgmv_onepass_kernel"
KERNEL_LAUNCHES = {BGMV_SHRINK: 2, "bgmv_multi": 3, ONEPASS: 1}


def _timed_eager(step, idx, lead_graph, steps, torch):
    """K steps of: replay lead_graph (long GPU work, so the host runs ahead),
    then the calls idx eagerly with a HIP event recorded before each call and
    after the last.  Returns the mean duration of each call in ms."""
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(len(idx) + 1)]
              for _ in range(steps)]
    torch.cuda.synchronize()
    for evs in evsets:
        lead_graph.replay()
        for e, i in zip(evs, idx):
            e.record()
            if step.calls[i][2]() != 0:
                raise RuntimeError(step.calls[i][0])
        evs[-1].record()
    torch.cuda.synchronize()
    return np.array([[evs[j].elapsed_time(evs[j + 1]) for j in range(len(idx))]
                     for evs in evsets]).mean(axis=0)


def _timed_graph(graph, lead_graph, steps, torch):
    """K times: replay lead_graph, then `graph` between two HIP events on the
    launch stream.  Returns the median replay duration in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        lead_graph.replay()
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))


def _timed_by_kernel(step, lead_graph, steps, torch):
    """Per-kernel launch duration: K times, replay lead_graph (so the host runs
    ahead), then for each kernel issue all of its launches of the step back to
    back, in step order, between two HIP events on the launch stream.  Returns
    {kernel: mean ms per launch}.  (The launches of one kernel run without the
    other stage in between; the fold's values are not used after this.)"""
    names = []
    for c in step.calls:
        if c[1] not in names:
            names.append(c[1])
    out = {}
    for kn in names:
        idx = [i for i, c in enumerate(step.calls) if c[1] == kn]
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            lead_graph.replay()
            e0.record()
            for i in idx:
                if step.calls[i][2]() != 0:
                    raise RuntimeError(step.calls[i][0])
            e1.record()
        torch.cuda.synchronize()
        out[kn] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) / len(idx)
    return out


def _read_once_fields(read_once, avg_launch_s):
    """For a fused kernel: its achieved rate and fraction of peak on the bytes
    the launch itself must move (read_once_bytes_per_launch), beside the
    per-call figure that `achieved` uses.  Empty for other kernels."""
    if not read_once or any(v is None for v in read_once):
        return {}
    b = sum(read_once) / len(read_once)
    a = b / avg_launch_s / 1e9
    return {"read_once_bytes_per_launch": int(b), "read_once_achieved": round(a, 1),
            "read_once_frac": round(a / HBM_PEAK_GBS, 4)}


def launch_floor_us(torch, dev, lead_graph, launches=200):
    """The empty-launch floor: a one-element fill kernel issued `launches`
    times back to back on the launch stream after a lead replay (the host
    ahead of the GPU), mean time per launch between two HIP events."""
    t = torch.zeros(1, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    lead_graph.replay()
    e0.record()
    for _ in range(launches):
        t.fill_(1.0)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / launches


COPY_BYTES = 256 << 20  # bytes read (and written) by one calibration copy


def copy_calibration(torch, dev):
    """Plain device-to-device copies of COPY_BYTES: the kernel reads and writes
    exactly that many bytes, so the ratio of a traffic counter's reading to
    COPY_BYTES calibrates that counter."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device=dev).fill_(7)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def run_gpu(args, traffic=True):
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if getattr(args, "copy_calibration", False):
        copy_calibration(torch, dev)
    wls = select_workloads(args.workload)
    step = Step(dev, wls)
    ncalls = len(step.calls)
    grouped = [i for i, c in enumerate(step.calls) if c[0].startswith("grouped.")]
    other = [i for i in range(ncalls) if i not in grouped]

    for _ in range(args.warmup):
        step.enqueue()
    torch.cuda.synchronize()

    cap_stream = torch.cuda.Stream()

    def capture(idx, parallel=False):
        return step.capture(idx, cap_stream, parallel)

    # the step as timed (independent calls on parallel branches), and sequential
    # captures that keep the GPU busy ahead of the per-call and per-kernel timing
    full = capture(range(ncalls), parallel=True)
    full_seq = capture(range(ncalls))
    g_other = capture(other) if other else None
    g_grouped = capture(grouped) if grouped else None
    for _ in range(3):
        full.replay()
        full_seq.replay()
    torch.cuda.synchronize()

    # timed region A: K replays of the whole step, back to back (an event after
    # each replay gives the per-replay spread; the wall clock gives the value)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        full.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rep_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    # timed regions B and C: every call timed by HIP events on the launch stream
    per_call_ms = np.zeros(ncalls)
    if grouped:
        lead = g_other if g_other is not None else g_grouped
        per_call_ms[grouped] = _timed_eager(step, grouped, lead, args.steps, torch)
    if other:
        lead = g_grouped if g_grouped is not None else g_other
        per_call_ms[other] = _timed_eager(step, other, lead, args.steps, torch)
    segs = [(i, i + 1) for i in range(ncalls)]
    seg_ms = per_call_ms
    # timed region D: each kernel's launches back to back (per-launch durations
    # for the kernel table and the roofline)
    kernel_ms = _timed_by_kernel(step, full_seq, args.steps, torch)
    floor_us = launch_floor_us(torch, dev, full_seq)

    ms_per_step = wall * 1e3 / args.steps
    # per kernel: launches, algorithmic bytes and flops per step, mean launch time
    kernels = {}
    for c in step.calls:
        k = kernels.setdefault(c[1], {"launches": 0, "bytes": 0, "flops": 0.0})
        k["launches"] += 1
        k["bytes"] += int(c[3])
        k["flops"] += float(c[4])
    for kn, k in kernels.items():
        k["ms"] = kernel_ms[kn] * k["launches"]
    dom_name, dom = max(kernels.items(), key=lambda kv: kv[1]["ms"])
    avg_launch_s = dom["ms"] / dom["launches"] * 1e-3
    bytes_per_launch = dom["bytes"] / dom["launches"]
    achieved = bytes_per_launch / avg_launch_s / 1e9
    traffic = measured_traffic(dom_name, args.workload) if traffic else None
    read_once = [step.read_once.get(c[0]) for c in step.calls if c[1] == dom_name]

    per_workload = {}
    for tag, _ in wls:
        sel = [j for j, (a, b) in enumerate(segs) if step.calls[a][0].startswith(tag + ".")]
        ms = float(seg_ms[sel].sum())
        calls = [c for (a, b) in (segs[j] for j in sel) for c in step.calls[a:b]]
        by = sum(c[3] for c in calls)
        fl = sum(c[4] for c in calls)
        rows = sum(c[5] for c in calls)
        launches = sum(KERNEL_LAUNCHES.get(c[1], 1) for c in calls)
        ent = {"ms": round(ms, 5), "calls": len(calls), "launches": launches,
               "launch_floor_ms": round(launches * floor_us * 1e-3, 5),
               "rows": rows, "rows_per_s": round(rows / (ms * 1e-3), 1),
               "algo_bytes": int(by), "gbs": round(by / (ms * 1e-3) / 1e9, 1),
               "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if tag == "grouped":
            ent["mfma_util"] = round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 5)
        # the workload alone as the step issues it (its independent calls on
        # parallel graph branches), after a replay of the rest of the step
        if len(wls) > 1:
            wsel = [a for a, _ in (segs[j] for j in sel)]
            lead = g_other if tag == "grouped" else g_grouped
            gms = _timed_graph(capture(wsel, parallel=True), lead, args.steps, torch)
            ent["graph"] = {"ms": round(gms, 5), "gbs": round(by / (gms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(by / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # the workload's dominant kernel against the HBM roofline (its launches
        # of this workload; per-launch time from the back-to-back timing)
        wk = {}
        for c in calls:
            k = wk.setdefault(c[1], [0, 0])
            k[0] += 1
            k[1] += int(c[3])
        kn, (nl, kb) = max(wk.items(), key=lambda kv: kernel_ms[kv[0]] * kv[1][0])
        kach = kb / nl / (kernel_ms[kn] * 1e-3) / 1e9
        ent["roofline"] = {"bound": "hbm", "kernel": kn, "achieved": round(kach, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(kach / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(kn, args.workload) if traffic else None,
                           "algo_bytes_per_launch": int(kb / nl),
                           "avg_launch_us": round(kernel_ms[kn] * 1e3, 3), "launches": nl,
                           **_read_once_fields([step.read_once.get(c[0]) for c in calls
                                                if c[1] == kn], kernel_ms[kn] * 1e-3)}
        per_workload[tag] = ent

    kern_out = {k: {"launches_per_step": v["launches"],
                    "avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                    "algo_bytes_per_launch": int(v["bytes"] / v["launches"]),
                    "gbs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)}
                for k, v in kernels.items()}
    return {
        "ms_per_step": ms_per_step,
        "replay_ms": {"median": round(float(np.median(rep_ms)), 5),
                      "p10": round(float(np.percentile(rep_ms, 10)), 5),
                      "p90": round(float(np.percentile(rep_ms, 90)), 5)},
        "ms_per_step_calls": float(seg_ms.sum()),
        "rows": step.rows,
        "bytes": step.bytes,
        "flops": step.flops,
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algo_bytes_per_launch": int(bytes_per_launch),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "launches_per_step": dom["launches"],
                     **_read_once_fields(read_once, avg_launch_s)},
        "kernels": kern_out,
        "per_workload": per_workload,
        "launch_floor_us": round(floor_us, 3),
    }


def run_model(args):
    """The multi-layer decode step: every layer's folds captured in one graph
    (q/k/v, o, gate, up, down; layers in order), the xa
    arena and workspaces shared by all layers, replayed K times.  Its adapter
    pools (about 1.3 GB) are five times the 256 MB MALL, so replays stream
    from HBM."""
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wls = model_workloads()
    step = Step(dev, wls)
    for _ in range(args.warmup):
        step.enqueue()
    torch.cuda.synchronize()
    g = step.capture(range(len(step.calls)), torch.cuda.Stream(), parallel=True)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        g.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rep_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    ms = wall * 1e3 / args.steps
    gbs = step.bytes / (ms * 1e-3) / 1e9
    pool_bytes = sum(a.A.nbytes + a.B.nbytes for _, wl in wls for c in wl.calls
                     for a in c.adapters)
    # The same graph with every row routed to the base model (seq_slot -1, the
    # graph-safe routing upload): every launch, routing scan and zero xa row
    # stays, no adapter byte is read and nothing folds, so the difference is
    # the cost of applying the adapters (the pages' no-apply lever, by routing).
    seqs = list(step.seqs.values())
    saved = [sq.clone() for sq in seqs]
    for sq in seqs:
        sq.fill_(-1)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    nf_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    for sq, v in zip(seqs, saved):
        sq.copy_(v)
    torch.cuda.synchronize()
    return {"workload": WORKLOAD_NAMES["model"], "layers": len(wls),
            "ms_per_step": round(ms, 5), "us_per_layer": round(ms * 1e3 / len(wls), 3),
            "replay_ms": {"median": round(float(np.median(rep_ms)), 5),
                          "p10": round(float(np.percentile(rep_ms, 10)), 5),
                          "p90": round(float(np.percentile(rep_ms, 90)), 5)},
            "rows_per_step": step.rows, "rows_per_s": round(step.rows / (ms * 1e-3), 1),
            "algo_bytes_per_step": int(step.bytes), "hbm_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "adapter_bytes": int(pool_bytes),
            "no_fold": {"ms_per_step": round(nf_ms, 5),
                        "what": "the same graph with every row routed to the base model "
                                "(seq_slot -1): launches, routing scans and zero xa rows, no "
                                "adapter read, no fold"}}


# ------------------------------------------------------------- CPU oracle ---

def _oracle_tasks(wls, cpu_rows):
    """The oracle's share of the step as independent tasks, with the install
    work (table packing) done here, outside any timing: each BGMV call, the
    gather fold, and the grouped projections in windows of at most 2048 sorted
    rows (the first cpu_rows rows of each).  Each task is (rows, fn)."""
    import oracle as O
    tasks = []
    for tag in ("attn", "ffn"):
        if tag not in wls:
            continue
        wl = wls[tag]
        for c in wl.calls:
            slots = O.pack_slots(c.adapters, c.max_loras, c.max_rank)

            def t(wl=wl, c=c, slots=slots):
                O.bgmv(slots, c.k_in, c.n_out, c.max_rank, wl.buffers[c.x_buf], c.x_row_stride,
                       wl.seq_slot, wl.n, wl.buffers[c.out_buf], c.out_offset, c.out_row_stride)
            tasks.append((wl.n, t))
    if "gather" in wls:
        wl = wls["gather"]
        pairs = O.pack_expert_pairs(wl.adapters, wl.max_loras, wl.num_experts, wl.max_rank)

        def t(wl=wl, pairs=pairs):
            O.moe_gather(pairs, wl.num_experts, wl.k_in, wl.n_out, wl.max_rank, wl.x.ravel(),
                         wl.k_in, wl.indices, wl.row_adapter, wl.top_k, wl.n_rows,
                         wl.base.ravel(), wl.n_out)
        tasks.append((wl.n_rows, t))
    if "grouped" in wls:
        wl = wls["grouped"]
        for p in wl.projections:
            pairs = O.pack_expert_pairs(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank)
            hi_all = min(cpu_rows, wl.te)
            for lo in range(0, hi_all, 2048):
                hi = min(lo + 2048, hi_all)

                def t(wl=wl, p=p, pairs=pairs, lo=lo, hi=hi):
                    O.moe_grouped(pairs, wl.num_experts, p.k_in, p.n_out, wl.max_rank,
                                  p.x.ravel(), p.k_in, p.x_gather, wl.num_tokens,
                                  wl.expert_offsets, wl.sorted_token_ids, wl.row_adapter, lo,
                                  hi, p.base.ravel(), p.n_out)
                tasks.append((hi - lo, t))
    return tasks


_TASKS = []


def _run_task(i):
    _TASKS[i][1]()
    return _TASKS[i][0]


def cpu_baseline(args):
    """The oracle, as it stands, on a bounded sample of the step (every BGMV
    and gather call in full, the first cpu_rows sorted rows of each grouped
    projection), timed on one core and on every core of the process's affinity
    mask (a pool of worker processes, one task at a time each).  BLAS is held
    to one thread per process.  Runs before the GPU is touched, so the pool's
    workers are plain forks of a process without a GPU context."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    wls = dict(select_workloads(args.workload))
    global _TASKS
    _TASKS = _oracle_tasks(wls, args.cpu_rows)
    rows = sum(r for r, _ in _TASKS)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _, fn in _TASKS:
            fn()
        dt1 = time.perf_counter() - t0
        cores = min(len(os.sched_getaffinity(0)), args.cpu_workers)
        with mp.get_context("fork").Pool(cores) as pool:
            pool.map(_run_task, range(min(cores, len(_TASKS))))  # workers up
            t0 = time.perf_counter()
            done = sum(pool.map(_run_task, range(len(_TASKS)), chunksize=1))
            dtn = time.perf_counter() - t0
    assert done == rows
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(rows / dtn, 1), "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} rows of the step (every BGMV and gather row, the first "
                      f"{args.cpu_rows} sorted rows of each grouped projection), "
                      f"{dtn:.2f} s on {cores} host cores ({model}) in worker processes; "
                      f"table packing outside the timing",
            "one_core": {"value": round(rows / dt1, 1), "seconds": round(dt1, 2)},
            "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="step", choices=list(WORKLOAD_NAMES))
    ap.add_argument("--cpu-rows", type=int, default=32768,
                    help="sorted rows per grouped projection in the cpu_baseline sample "
                         "(the default covers the whole step)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="most worker processes of the all-cores oracle timing")
    ap.add_argument("--no-unrouted", action="store_true",
                    help="with the default step: skip the separate unrouted-path measurement")
    ap.add_argument("--no-model", action="store_true",
                    help="with the default step: skip the multi-layer decode step")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print a markdown summary of rocprofv3 output directories and exit")
    ap.add_argument("--bench-json", help="with --summarize: a bench.py output line to include")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run plain device copies of COPY_BYTES (256 MiB) each, so that "
                         "a counter run sees the counters of a copy of known size")
    args = ap.parse_args()
    if args.summarize:
        print(summarize(args.summarize, args.bench_json, args.workload))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the routed fold has no multi-GPU path in this "
              "library (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    # the oracle's timing first, before this process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(args)
    g = run_gpu(args)
    rows_per_s = g["rows"] / (g["ms_per_step"] * 1e-3)
    gbs = g["bytes"] / (g["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64; shapes and routing of the routed-LoRA workloads)",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "rows_per_step": g["rows"],
                   "algo_bytes_per_step": int(g["bytes"]), "flops_per_step": int(g["flops"])},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "replay_ms": g["replay_ms"],
        "ms_per_step_calls": round(g["ms_per_step_calls"], 5),
        "launch_floor_us": g["launch_floor_us"],
        "roofline": g["roofline"],
        "cpu_baseline": cpu,
        "kernels": g["kernels"],
        "per_workload": g["per_workload"],
    }
    if args.workload == "step" and not args.no_model:
        # The multi-layer decode step, measured on its own; not part of `value`.
        line["decode_model"] = run_model(args)
    if args.workload == "step" and not args.no_unrouted:
        # The unrouted single-adapter path (apply_lora_delta), measured the same
        # way on its own prefill workload; not part of the step or of `value`.
        ua = argparse.Namespace(**{**vars(args), "workload": "lora", "copy_calibration": False})
        u = run_gpu(ua)
        ugbs = u["bytes"] / (u["ms_per_step"] * 1e-3) / 1e9
        line["unrouted"] = {
            "workload": WORKLOAD_NAMES["lora"], "ms_per_pass": round(u["ms_per_step"], 5),
            "rows_per_pass": u["rows"], "rows_per_s": round(u["rows"] / (u["ms_per_step"] * 1e-3), 1),
            "algo_bytes_per_pass": int(u["bytes"]), "hbm_gbs": round(ugbs, 1),
            "hbm_frac": round(ugbs / HBM_PEAK_GBS, 4),
            "mfma_util": round(u["flops"] / (u["ms_per_step"] * 1e-3) / 1e12
                               / BF16_MFMA_PEAK_TFLOPS, 5),
            "roofline": u["roofline"], "kernels": u["kernels"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
