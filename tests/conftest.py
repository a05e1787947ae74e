import json
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The stated tolerances and the configurations of the parity tests whose
# comparisons are summarised per configuration.
CONFIG_TESTS = {
    "test_bgmv_tiny_config": "tiny routed BGMV (n=4, k_in=n_out=256, r=8)",
    "test_bgmv_attn_decode_config": "attention decode BGMV (Qwen3-8B q/k/v/o, n=64, r=16)",
    "test_bgmv_ffn_decode_config": "FFN decode BGMV (n=256, 4096x12288, r=64)",
    "test_moe_gather[config]": "MoE decode gather fold (32 tokens x top-8, 768->2048, r=16)",
    "test_moe_gather[config_seed103]":
        "MoE decode gather fold (32 tokens x top-8, 768->2048, r=16)",
    "test_moe_grouped_full_config": "MoE grouped prefill (te=32768, cap 8192, r=32), every row",
}


def _seed_note(name):
    """The full-size configurations also run at a second seed (workload seed
    index 100 above the configuration's own); their rows are listed apart."""
    m = re.search(r"seed(\d+)\]$", name)
    return ", second seed" if m and int(m.group(1)) >= 100 else ""


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _parity_markdown(recs):
    lines = ["Parity counts of the GPU tests against the oracle, per comparison.", "",
             "Stated rule: xa and delta within 1 BF16 ulp; folded outputs within "
             "max(2 BF16 ulp, 1e-3 absolute); routing and base rows bit-exact.  "
             "`widened` counts the elements accepted only under the derived fp32 "
             "summation bound (xa/delta, capped at 1e-3 of the elements) or the "
             "derived fold bound (outputs, capped at 1e-4 of the outputs).", ""]
    per_cfg = {}
    for r in recs:
        name = r["test"].split("::")[-1]
        cfg = CONFIG_TESTS.get(name) or CONFIG_TESTS.get(name.split("[")[0])
        if cfg is None:
            continue
        c = per_cfg.setdefault((cfg + _seed_note(name), r["kind"]), [0, 0, 0, 0])
        c[0] += r["elements"]
        c[1] += r["bit_exact"]
        c[2] += r["within_stated"]
        c[3] += r["widened"]
    lines += ["Per configuration:", "",
              "| configuration | compared | elements | bit-exact | within the stated rule, "
              "not bit-exact | widened |", "|---|---|---|---|---|---|"]
    for (cfg, kind), (n, ex, w, wd) in sorted(per_cfg.items()):
        what = "xa / delta" if kind == "xa" else "folded outputs"
        lines.append(f"| {cfg} | {what} | {n} | {ex} | {w} | {wd} |")
    tot = {}
    for r in recs:
        t = tot.setdefault(r["kind"], [0, 0, 0, 0])
        t[0] += r["elements"]
        t[1] += r["bit_exact"]
        t[2] += r["within_stated"]
        t[3] += r["widened"]
    lines += ["", "All GPU comparisons of the run:", "",
              "| compared | elements | bit-exact | within the stated rule, not bit-exact | "
              "widened |", "|---|---|---|---|---|"]
    for kind, (n, ex, w, wd) in sorted(tot.items()):
        what = "xa / delta" if kind == "xa" else "folded outputs"
        lines.append(f"| {what} | {n} | {ex} | {w} | {wd} |")
    wide = [r for r in recs if r["widened"]]
    lines += ["", f"Comparisons with widened elements: {len(wide)} of {len(recs)}.", ""]
    if wide:
        lines += ["| test | comparison | elements | widened |", "|---|---|---|---|"]
        for r in wide:
            lines.append(f"| {r['test'].split('::')[-1]} | {r['label']} | {r['elements']} | "
                         f"{r['widened']} |")
    return "\n".join(lines) + "\n"


def pytest_sessionfinish(session, exitstatus):
    out = os.environ.get("RLD_PARITY_OUT")
    if not out:
        return
    mod = sys.modules.get("gpu_util")
    recs = getattr(mod, "PARITY_RECORDS", []) if mod else []
    if not recs:
        return
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "parity_counts.json"), "w") as fh:
        json.dump(recs, fh, indent=0)
    with open(os.path.join(out, "parity_counts.md"), "w") as fh:
        fh.write(_parity_markdown(recs))


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
