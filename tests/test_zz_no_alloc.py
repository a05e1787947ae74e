"""rld_bgmv_noalloc (the routed BGMV fold with its xa arena and k-split partials
in the library's fixed per-GPU scratch, for callers that cannot allocate)
against rld_bgmv with caller buffers: the same bits, on two calls in a row
(the second smaller), and under HIP graph replay with new routing."""
import numpy as np
import pytest
import torch

import routed_lora_delta_amd as R
import workloads as W
from gpu_util import GUARD, BgmvRun, compare_bgmv, require_gpu, say
from routed_lora_delta_amd.pool import from_device_u16

pytestmark = pytest.mark.gpu


def _noalloc_run(wl, dev):
    """Every call of the workload through rld_bgmv_noalloc on fresh buffers."""
    run = BgmvRun(wl, dev)
    for i, c in enumerate(wl.calls):
        R.check(R.rld_bgmv_noalloc(run.routes[i].route, run.bufs[c.x_buf].ptr(), c.x_row_stride,
                                   run.seq, wl.n, run.bufs[c.out_buf].ptr(c.out_offset),
                                   c.out_row_stride), f"rld_bgmv_noalloc {c.module}")
    torch.cuda.synchronize()
    return run


def test_noalloc_equals_bgmv_two_calls():
    """First the FFN decode folds (n = 256, gate/up 4096 -> 12288 and down
    12288 -> 4096 at rank 64: 24-chunk k split), then a smaller call (n = 37,
    k_in 4096 -> 1032 at rank 16) on the same scratch: each output bit-identical
    to rld_bgmv with caller buffers, and the first against the oracle."""
    dev = require_gpu()
    big = W.bgmv_ffn_decode()
    small = W.bgmv_custom(5, 37, 4096, 1032, 16, 16, (8, 16), base_frac=0.1)
    for wl in (big, small):
        say(f"case: noalloc {wl.name} n={wl.n}")
        want = BgmvRun(wl, dev)
        want.run_all(keep_xa=False)
        got = _noalloc_run(wl, dev)
        for k, b in want.outputs().items():
            assert np.array_equal(got.outputs()[k], b), f"{wl.name}: buffer {k}"
    # the first call's outputs meet the oracle too (compare_bgmv needs each call's xa)
    run = BgmvRun(big, dev)
    run.run_all()
    compare_bgmv(run, "noalloc reference")


def test_noalloc_graph_replay_new_routing():
    """rld_bgmv_noalloc captured into a HIP graph (the case it exists for) and
    replayed with a new seq_slot before each replay: every replay equals an
    eager rld_bgmv with caller buffers on the same routing."""
    dev = require_gpu()
    wl = W.bgmv_custom(6, 96, 4096, 4096, 16, 16, (8, 16), base_frac=0.1)
    c = wl.calls[0]
    say("case: noalloc graph replay")
    run = BgmvRun(wl, dev)
    # one eager call first, so the scratch address lookup happens outside capture
    R.check(R.rld_bgmv_noalloc(run.routes[0].route, run.bufs[c.x_buf].ptr(), c.x_row_stride,
                               run.seq, wl.n, run.bufs[c.out_buf].ptr(), c.out_row_stride),
            "eager rld_bgmv_noalloc")
    torch.cuda.synchronize()
    pristine = {k: torch.from_numpy(np.ascontiguousarray(v).ravel().view(np.int16)).to(dev)
                for k, v in wl.buffers.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        R.check(R.rld_bgmv_noalloc(run.routes[0].route, run.bufs[c.x_buf].ptr(), c.x_row_stride,
                                   run.seq, wl.n, run.bufs[c.out_buf].ptr(), c.out_row_stride, s),
                "captured rld_bgmv_noalloc")
    rng = np.random.default_rng(61)
    for rep in range(3):
        seq = rng.integers(-1, 17, size=wl.n).astype(np.int32)
        run.seq.copy_(torch.from_numpy(seq))
        for k, b in run.bufs.items():
            b.t[GUARD:GUARD + b.size].copy_(pristine[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = BgmvRun(W.BgmvWorkload(**{**wl.__dict__, "seq_slot": seq}), dev)
        ref.run_all(keep_xa=False)
        got = from_device_u16(run.bufs[c.out_buf].t)
        want = from_device_u16(ref.bufs[c.out_buf].t)
        assert np.array_equal(got, want), f"replay {rep}"
        _ = torch.ones(1 << 20, device=dev).sum().item()  # eager work between replays
