"""CPU oracle of the routed LoRA delta: TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The library never does.
"""
from .rld_oracle import *  # noqa: F401,F403
from .rld_oracle import (BF16_MAX, M_TILE, SlotWeights, bf16_to_f32, bf16_to_f64,  # noqa: F401
                         bgmv, expert_owner, f16_to_bf16, fold_row, gather_row_token,
                         grouped_down_wc, grouped_down_windows, lora_delta, moe_gather,
                         moe_grouped,
                         pack_expert_pairs, pack_expert_tables, pack_slots, pad_adapter,
                         round_bf16, scale_for)
