"""Adapter pools and route tables on the device (install time).

The padded A and B of every adapter of one module live in a single device
buffer (each tensor 256-byte aligned).  Padding goes through
rld_pad_adapter_host and the tables through rld_route_pack /
rld_moe_tables_pack (the C ABI); torch only provides the device memory the
results are copied into.  Objects keep their tensors alive, so the addresses
in the tables stay valid for the object's lifetime.
"""
from __future__ import annotations

import ctypes
from typing import Sequence

import numpy as np
import torch

from . import (check, rld_adapter_entry, rld_f16_to_bf16_host, rld_grouped_windows,
               rld_moe_route, rld_moe_tables_pack, rld_pad_adapter_host, rld_pair, rld_route,
               rld_route_pack, rld_scale)

_ALIGN_ELEMS = 128  # 256 bytes of BF16


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def install_peft_pair(a_f16: np.ndarray, b_f16: np.ndarray, rank: int, k_in: int, n_out: int,
                      max_rank: int, alpha: float, use_rslora: bool):
    """Host side of installing one PEFT module stored as F16 (lora_A [rank,
    k_in], lora_B [n_out, rank]): F16 -> BF16 (rld_f16_to_bf16_host), padded to
    the pool layout (rld_pad_adapter_host) and the fp32 scale (rld_scale).
    Returns (A [max_rank, k_in], B [n_out, max_rank] BF16 bits, scale)."""
    a16 = np.ascontiguousarray(a_f16, np.uint16).reshape(rank, k_in)
    b16 = np.ascontiguousarray(b_f16, np.uint16).reshape(n_out, rank)
    a_bf, b_bf = np.empty_like(a16), np.empty_like(b16)
    check(rld_f16_to_bf16_host(a16.ravel(), a_bf.ravel(), a16.size), "rld_f16_to_bf16_host")
    check(rld_f16_to_bf16_host(b16.ravel(), b_bf.ravel(), b16.size), "rld_f16_to_bf16_host")
    a_pad = np.empty((max_rank, k_in), np.uint16)
    b_pad = np.empty((n_out, max_rank), np.uint16)
    check(rld_pad_adapter_host(a_bf, b_bf, rank, k_in, n_out, max_rank, a_pad, b_pad),
          "rld_pad_adapter_host")
    sc = ctypes.c_float()
    check(rld_scale(alpha, rank, use_rslora, ctypes.byref(sc)), "rld_scale")
    return a_pad, b_pad, np.float32(sc.value)


def to_device_u16(arr: np.ndarray, device) -> torch.Tensor:
    """uint16 BF16 bits -> device int16 tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)


def from_device_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


class _Pool:
    def __init__(self, adapters: Sequence, k_in: int, n_out: int, max_rank: int, device):
        self.k_in, self.n_out, self.max_rank = k_in, n_out, max_rank
        a_elems = _round_up(max_rank * k_in, _ALIGN_ELEMS)
        b_elems = _round_up(n_out * max_rank, _ALIGN_ELEMS)
        total = max(1, len(adapters)) * (a_elems + b_elems)
        host = np.zeros(total, np.uint16)
        offs = []
        for i, ad in enumerate(adapters):
            oa = i * (a_elems + b_elems)
            ob = oa + a_elems
            A = np.ascontiguousarray(ad.A, np.uint16)
            B = np.ascontiguousarray(ad.B, np.uint16)
            check(rld_pad_adapter_host(A, B, ad.rank, k_in, n_out, max_rank,
                                       host.ctypes.data + 2 * oa, host.ctypes.data + 2 * ob),
                  "rld_pad_adapter_host")
            offs.append((oa, ob))
        self.buf = to_device_u16(host, device)
        base = self.buf.data_ptr()
        self.entries = (rld_adapter_entry * max(1, len(adapters)))()
        for i, (ad, (oa, ob)) in enumerate(zip(adapters, offs)):
            e = self.entries[i]
            e.slot = ad.slot
            e.expert = -1 if ad.expert is None else ad.expert
            e.a_addr = base + 2 * oa
            e.b_addr = base + 2 * ob
            e.rank = ad.rank
            e.alpha = ad.alpha
            e.use_rslora = int(ad.use_rslora)
        self.n_entries = len(adapters)
        self.nbytes = 2 * total


class DenseRoute:
    """Slot-keyed route of one module (LoraRoute): tables [max_loras]."""

    def __init__(self, adapters: Sequence, max_loras: int, max_rank: int, k_in: int, n_out: int,
                 device="cuda"):
        self.pool = _Pool(adapters, k_in, n_out, max_rank, device)
        a = np.zeros(max_loras, np.uint64)
        b = np.zeros(max_loras, np.uint64)
        s = np.zeros(max_loras, np.float32)
        check(rld_route_pack(self.pool.entries, self.pool.n_entries, max_loras, max_rank, a, b, s),
              "rld_route_pack")
        self.a_host, self.b_host, self.scale_host = a, b, s
        self.a_table = torch.from_numpy(a.view(np.int64).copy()).to(device)
        self.b_table = torch.from_numpy(b.view(np.int64).copy()).to(device)
        self.scale_table = torch.from_numpy(s.copy()).to(device)
        self.route = rld_route(self.a_table.data_ptr(), self.b_table.data_ptr(),
                               self.scale_table.data_ptr(), max_loras, k_in, n_out, max_rank)

    def set_table_entry(self, slot: int, a_addr=None, b_addr=None):
        """Overwrite one table entry on the device (tests of the 0 = base-only rule)."""
        if a_addr is not None:
            self.a_table[slot] = int(np.int64(np.uint64(a_addr)))
        if b_addr is not None:
            self.b_table[slot] = int(np.int64(np.uint64(b_addr)))


class SinglePair:
    """One adapter module without routing (LoraPair): the pair packed on slot 0 of
    a one-slot route, so the same pool serves the unrouted and the routed calls."""

    def __init__(self, adapter, max_rank: int, k_in: int, n_out: int, device="cuda"):
        assert adapter.slot == 0
        self.route = DenseRoute([adapter], 1, max_rank, k_in, n_out, device)
        r = self.route
        self.pair = rld_pair(int(r.a_host[0]), int(r.b_host[0]), float(r.scale_host[0]), k_in,
                             n_out, max_rank)


class MoeRoute:
    """Expert routing tables of one MoE projection: [max_loras][num_experts]."""

    def __init__(self, adapters: Sequence, max_loras: int, num_experts: int, max_rank: int,
                 k_in: int, n_out: int, device="cuda"):
        self.pool = _Pool(adapters, k_in, n_out, max_rank, device)
        n = max_loras * num_experts
        a = np.zeros(n, np.uint64)
        b = np.zeros(n, np.uint64)
        s = np.zeros(n, np.float32)
        check(rld_moe_tables_pack(self.pool.entries, self.pool.n_entries, max_loras, num_experts,
                                  max_rank, a, b, s), "rld_moe_tables_pack")
        self.a_table = torch.from_numpy(a.view(np.int64).copy()).to(device)
        self.b_table = torch.from_numpy(b.view(np.int64).copy()).to(device)
        self.scale_table = torch.from_numpy(s.copy()).to(device)
        self.route = rld_moe_route(self.a_table.data_ptr(), self.b_table.data_ptr(),
                                   self.scale_table.data_ptr(), max_loras, num_experts, k_in,
                                   n_out, max_rank)


def grouped_windows(total_rows: int, cap: int):
    """The [start, end) launch windows of at most cap rows that cover
    0..total_rows, from the library's rld_grouped_windows."""
    n = max(1, -(-total_rows // cap)) if cap > 0 else 1
    starts = np.zeros(n, np.uint32)
    ends = np.zeros(n, np.uint32)
    cnt = ctypes.c_uint32(0)
    check(rld_grouped_windows(total_rows, cap, starts, ends, n, ctypes.byref(cnt)),
          "rld_grouped_windows")
    return [(int(a), int(b)) for a, b in zip(starts[:cnt.value], ends[:cnt.value])]
