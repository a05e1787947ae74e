"""The multi-layer decode step on the GPU ("Function apply_lora_bgmv",
GRAPH-SAFE paragraph: the per-layer tables and the xa arena are fixed; only the
contents of seq_slot change from step to step): 36 decoder layers of Qwen3-8B
shapes, every projection adapted with the layer's own pools, captured once as
one HIP graph with one xa arena and one workspace per branch shared by every
layer.  Before each replay the batch's seq_slot gets a new routing."""
import numpy as np
import pytest
import torch

import routed_lora_delta_amd as R
import workloads as W
from gpu_util import compare_bgmv_outputs, require_gpu, say
from routed_lora_delta_amd.pool import from_device_u16

pytestmark = pytest.mark.gpu

SAMPLED = (0, 17, 35)


def test_model_step_graph_new_routing_each_replay():
    """Each replay, with new seq_slot contents (a different batch of slots and
    base rows), gives exactly the bits of the same calls issued eagerly on that
    routing, for every buffer of every layer; layers 0, 17 and 35 of each
    replay also meet the oracle (outputs within tolerance, base rows and
    everything outside the folded regions bit-exact)."""
    import bench
    dev = require_gpu()
    wls = bench.model_workloads()
    assert len(wls) == 36
    say("case: model step, 36 layers, building")
    step = bench.Step(dev, wls)
    (seq,) = step.seqs.values()  # the one routing buffer every layer reads
    pristine = {k: t.clone() for k, t in step.outputs.items()}
    stream = torch.cuda.Stream()
    g = step.capture(range(len(step.calls)), stream, parallel=True)
    rng = np.random.default_rng(97)
    for rep in range(3):
        routing = rng.integers(-1, 18, size=len(wls[0][1].seq_slot)).astype(np.int32)
        say(f"case: model step replay {rep}, {int((routing < 0).sum())} base rows, "
            f"{int((routing >= 16).sum())} slots past max_loras")
        seq.copy_(torch.from_numpy(routing))
        for k, t in step.outputs.items():
            t.copy_(pristine[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: t.clone() for k, t in step.outputs.items()}
        # the same calls, eagerly, on the same routing
        for k, t in step.outputs.items():
            t.copy_(pristine[k])
        step.enqueue()
        torch.cuda.synchronize()
        for k, t in step.outputs.items():
            assert torch.equal(got[k], t), f"replay {rep}: {k} differs from the eager calls"
        for li in SAMPLED:
            tag, wl = wls[li]
            wl_r = W.BgmvWorkload(**{**wl.__dict__, "seq_slot": routing})
            outs = {k: from_device_u16(got[f"{tag}.{k}"]) for k in wl.buffers}
            compare_bgmv_outputs(wl_r, outs, f"replay {rep} {tag}")
        _ = torch.ones(1 << 20, device=dev).sum().item()  # eager work between replays
