"""Python binding of librld.so, the routed LoRA delta library for gfx950.

Argument marshalling only: every function below has the name of the C entry
point it calls (include/rld.h) and forwards its arguments unchanged.  Pointer
arguments accept an int address, None, or any object with ``data_ptr()``
(a torch tensor); ``stream`` accepts an int handle, a torch stream, or None
for torch's current stream.  Entry points return the library's status code;
``check()`` turns a non-zero status into an ``RldError``.

There is no fallback: if librld.so has not been built, importing this package
raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_float, c_int, c_int32, c_size_t, c_uint32, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librld.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rld.h")

RLD_OK, RLD_EINVAL, RLD_EALIGN, RLD_EUNSUPPORTED, RLD_ELAUNCH, RLD_ENOSPACE = 0, -1, -2, -3, -4, -5
RLD_MAX_RANK = 128
RLD_NOALLOC_SCRATCH_BYTES = 8 << 20
RLD_M_TILE = 64

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "or python routed_lora_delta_amd/build.py")

# The library must run on the same HIP runtime instance as the framework whose
# device memory and streams it is handed.  torch ships its own libamdhip64;
# loading it first makes librld.so's libamdhip64.so.7 dependency resolve to
# that copy.  Loaded the other way round, the process would hold two HIP
# runtimes, and the second to open the GPU finds no device.
try:
    import torch  # noqa: F401
except ImportError:  # standalone use: librld.so's own ROCm runtime
    pass

_lib = ctypes.CDLL(LIB_PATH)


class RldError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {rld_status_string(status)} ({status})"
                         f"{', hip error %d' % rld_last_hip_error() if status == RLD_ELAUNCH else ''}")


class rld_route(ctypes.Structure):
    _fields_ = [("a_table", c_void_p), ("b_table", c_void_p), ("scale_table", c_void_p),
                ("max_loras", c_uint32), ("k_in", c_uint32), ("n_out", c_uint32),
                ("max_rank", c_uint32)]


class rld_pair(ctypes.Structure):
    _fields_ = [("a", c_void_p), ("b", c_void_p), ("scale", c_float), ("k_in", c_uint32),
                ("n_out", c_uint32), ("max_rank", c_uint32)]


class rld_moe_route(ctypes.Structure):
    _fields_ = [("a_table", c_void_p), ("b_table", c_void_p), ("scale_table", c_void_p),
                ("max_loras", c_uint32), ("num_experts", c_uint32), ("k_in", c_uint32),
                ("n_out", c_uint32), ("max_rank", c_uint32)]


class rld_adapter_entry(ctypes.Structure):
    _fields_ = [("slot", c_uint32), ("expert", c_int32), ("a_addr", c_uint64),
                ("b_addr", c_uint64), ("rank", c_uint32), ("alpha", c_float),
                ("use_rslora", c_int32)]


_P = c_void_p
_R = POINTER(rld_route)
_M = POINTER(rld_moe_route)
_L = POINTER(rld_pair)
_E = POINTER(rld_adapter_entry)
_u32p = POINTER(c_uint32)

_SIGS = {
    "rld_scale": (c_int, [c_float, c_uint32, c_int, POINTER(c_float)]),
    "rld_pad_adapter_host": (c_int, [_P, _P, c_uint32, c_uint32, c_uint32, c_uint32, _P, _P]),
    "rld_route_pack": (c_int, [_E, c_size_t, c_uint32, c_uint32, _P, _P, _P]),
    "rld_moe_tables_pack": (c_int, [_E, c_size_t, c_uint32, c_uint32, c_uint32, _P, _P, _P]),
    "rld_pack_expert_tables": (c_int, [_P, _P, _P, _P, c_size_t, c_uint32, _P, _P, _P, _u32p]),
    "rld_grouped_windows": (c_int, [c_uint32, c_uint32, _P, _P, c_uint32, _u32p]),
    "rld_grouped_wc": (c_uint32, [c_uint32, c_uint32]),
    "rld_gather_row_token": (c_uint32, [c_uint32, c_uint32]),
    "rld_gather_grids": (c_int, [c_uint32, c_uint32, c_uint32, _P]),
    "rld_bgmv_workspace_bytes": (c_size_t, [c_uint32, c_uint32, c_uint32, c_uint32]),
    "rld_bgmv_shrink": (c_int, [_R, _P, c_uint32, _P, c_uint32, _P, _P, c_size_t, _P]),
    "rld_bgmv_expand_fold": (c_int, [_R, _P, _P, c_uint32, _P, c_uint32, _P]),
    "rld_bgmv": (c_int, [_R, _P, c_uint32, _P, c_uint32, _P, c_uint32, _P, _P, c_size_t, _P]),
    "rld_bgmv_noalloc": (c_int, [_R, _P, c_uint32, _P, c_uint32, _P, c_uint32, _P]),
    "rld_bgmv_launches": (c_int, [_P, c_uint32, c_uint32]),
    "rld_bgmv_multi_workspace_bytes": (c_size_t, [c_uint32, c_uint32, c_uint32, c_uint32]),
    "rld_bgmv_multi": (c_int, [_P, c_uint32, _P, c_uint32, _P, c_uint32, _P, _P, _P, _P,
                               c_size_t, _P]),
    "rld_f16_to_bf16_host": (c_int, [_P, _P, c_size_t]),
    "rld_lora_workspace_bytes": (c_size_t, [c_uint32, c_uint32, c_uint32]),
    "rld_lora_shrink": (c_int, [_L, _P, c_uint32, c_uint32, _P, _P, c_size_t, _P]),
    "rld_lora_expand_fold": (c_int, [_L, _P, c_uint32, _P, c_uint32, _P]),
    "rld_lora_delta": (c_int, [_L, _P, c_uint32, c_uint32, _P, c_uint32, _P, _P, c_size_t, _P]),
    "rld_moe_gather_shrink": (c_int, [_M, _P, c_uint32, _P, _P, c_uint32, c_uint32, _P, _P]),
    "rld_moe_gather_expand_fold": (c_int, [_M, _P, _P, _P, c_uint32, c_uint32, _P, c_uint32,
                                           _P]),
    "rld_moe_gather": (c_int, [_M, _P, c_uint32, _P, _P, c_uint32, c_uint32, _P, c_uint32, _P,
                               _P]),
    "rld_moe_grouped_workspace_bytes": (c_size_t, [c_uint32, c_uint32, c_uint32, c_uint32,
                                                   c_uint32]),
    "rld_moe_grouped_shrink": (c_int, [_M, _P, c_uint32, c_int, c_uint32, _P, c_uint32, _P, _P,
                                       c_uint32, c_uint32, _P, c_uint32, _P, c_size_t, _P]),
    "rld_moe_grouped_expand_fold": (c_int, [_M, _P, c_uint32, _P, c_uint32, _P, _P, c_uint32,
                                            c_uint32, _P, c_uint32, _P]),
    "rld_moe_grouped": (c_int, [_M, _P, c_uint32, c_int, c_uint32, _P, c_uint32, _P, _P,
                                c_uint32, c_uint32, _P, c_uint32, _P, c_uint32, _P, c_size_t,
                                _P]),
    "rld_moe_grouped_pair": (c_int, [_M, _M, _P, c_uint32, c_int, c_uint32, _P, c_uint32, _P,
                                     _P, c_uint32, c_uint32, _P, c_uint32, _P, c_uint32, _P, _P,
                                     c_uint32, _P, c_size_t, _P]),
    "rld_status_string": (ctypes.c_char_p, [c_int]),
    "rld_last_hip_error": (c_int, []),
    "rld_version": (ctypes.c_char_p, []),
}

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def header_symbols():
    """Names of the functions include/rld.h declares."""
    with open(HEADER) as f:
        txt = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(rld_\w+)\(", txt, re.M)))


def ptr(obj) -> int | None:
    """Marshal a pointer argument: int address, None, or an object with data_ptr()."""
    if obj is None:
        return None
    if isinstance(obj, int):
        return obj
    if hasattr(obj, "data_ptr"):
        return obj.data_ptr()
    if hasattr(obj, "ctypes"):  # numpy array (host helpers)
        return obj.ctypes.data
    raise TypeError(f"cannot pass {type(obj)} as a pointer")


def stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def check(status: int, what: str = "rld") -> None:
    if status != RLD_OK:
        raise RldError(status, what)


# ------------------------------------------------------------------ host ----

def rld_scale(alpha, rank, use_rslora, out):
    return _lib.rld_scale(alpha, rank, int(use_rslora), out)


def rld_pad_adapter_host(a, b, rank, k_in, n_out, max_rank, a_pad, b_pad):
    return _lib.rld_pad_adapter_host(ptr(a), ptr(b), rank, k_in, n_out, max_rank, ptr(a_pad),
                                     ptr(b_pad))


def rld_route_pack(entries, n_entries, max_loras, max_rank, a_out, b_out, scale_out):
    return _lib.rld_route_pack(entries, n_entries, max_loras, max_rank, ptr(a_out), ptr(b_out),
                               ptr(scale_out))


def rld_moe_tables_pack(entries, n_entries, max_loras, num_experts, max_rank, a_out, b_out,
                        scale_out):
    return _lib.rld_moe_tables_pack(entries, n_entries, max_loras, num_experts, max_rank,
                                    ptr(a_out), ptr(b_out), ptr(scale_out))


def rld_pack_expert_tables(expert_ids, a_addrs, b_addrs, scales, n_entries, cap, a_out, b_out,
                           scale_out, n_experts_out):
    return _lib.rld_pack_expert_tables(ptr(expert_ids), ptr(a_addrs), ptr(b_addrs), ptr(scales),
                                       n_entries, cap, ptr(a_out), ptr(b_out), ptr(scale_out),
                                       n_experts_out)


def rld_grouped_windows(total_rows, cap, starts, ends, max_windows, count):
    return _lib.rld_grouped_windows(total_rows, cap, ptr(starts), ptr(ends), max_windows, count)


def rld_grouped_wc(row_offset, row_end):
    return _lib.rld_grouped_wc(row_offset, row_end)


def rld_gather_row_token(row, top_k):
    return _lib.rld_gather_row_token(row, top_k)


def rld_gather_grids(max_rank, n_out, n_rows, out):
    return _lib.rld_gather_grids(max_rank, n_out, n_rows, ptr(out))


def rld_bgmv_workspace_bytes(n, k_in, max_rank, max_loras):
    return _lib.rld_bgmv_workspace_bytes(n, k_in, max_rank, max_loras)


def rld_status_string(status):
    return _lib.rld_status_string(status).decode()


def rld_last_hip_error():
    return _lib.rld_last_hip_error()


def rld_version():
    return _lib.rld_version().decode()


# ---------------------------------------------------------------- device ----

def rld_bgmv_shrink(route, x, x_row_stride, seq_slot, n, xa, workspace, workspace_bytes,
                    stream=None):
    return _lib.rld_bgmv_shrink(ctypes.byref(route), ptr(x), x_row_stride, ptr(seq_slot), n,
                                ptr(xa), ptr(workspace), workspace_bytes, stream_handle(stream))


def rld_bgmv_expand_fold(route, xa, seq_slot, n, base_out, out_row_stride, stream=None):
    return _lib.rld_bgmv_expand_fold(ctypes.byref(route), ptr(xa), ptr(seq_slot), n,
                                     ptr(base_out), out_row_stride, stream_handle(stream))


def rld_bgmv(route, x, x_row_stride, seq_slot, n, base_out, out_row_stride, xa, workspace,
             workspace_bytes, stream=None):
    return _lib.rld_bgmv(ctypes.byref(route), ptr(x), x_row_stride, ptr(seq_slot), n,
                         ptr(base_out), out_row_stride, ptr(xa), ptr(workspace), workspace_bytes,
                         stream_handle(stream))


def rld_bgmv_launches(routes, n):
    """Launches of rld_bgmv (one route) or rld_bgmv_multi (a list of routes)."""
    if not isinstance(routes, (list, tuple)):
        routes = [routes]
    arr = (ctypes.c_void_p * len(routes))(*[ctypes.addressof(r) for r in routes])
    return _lib.rld_bgmv_launches(ctypes.cast(arr, c_void_p), len(routes), n)


def rld_bgmv_noalloc(route, x, x_row_stride, seq_slot, n, base_out, out_row_stride, stream=None):
    return _lib.rld_bgmv_noalloc(ctypes.byref(route), ptr(x), x_row_stride, ptr(seq_slot), n,
                                 ptr(base_out), out_row_stride, stream_handle(stream))


def rld_bgmv_multi_workspace_bytes(n, k_in, max_rank, nroutes):
    return _lib.rld_bgmv_multi_workspace_bytes(n, k_in, max_rank, nroutes)


def rld_bgmv_multi(routes, x, x_row_stride, seq_slot, n, base_out, out_row_stride, xa,
                   workspace, workspace_bytes, stream=None, nroutes=None):
    """routes, base_out, out_row_stride, xa: sequences with one entry per route
    (marshalled into the host arrays the call takes); nroutes defaults to
    len(routes)."""
    k = len(routes)
    nr = k if nroutes is None else nroutes
    rt = (c_void_p * max(k, 1))(*[ctypes.addressof(r) for r in routes])
    bo = (c_void_p * max(k, 1))(*[ptr(b) for b in base_out])
    os_ = (c_uint32 * max(k, 1))(*out_row_stride)
    xs = (c_void_p * max(k, 1))(*[ptr(v) for v in xa])
    return _lib.rld_bgmv_multi(ctypes.cast(rt, c_void_p), nr, ptr(x), x_row_stride,
                               ptr(seq_slot), n, ctypes.cast(bo, c_void_p),
                               ctypes.cast(os_, c_void_p), ctypes.cast(xs, c_void_p),
                               ptr(workspace), workspace_bytes, stream_handle(stream))


def rld_f16_to_bf16_host(src, dst, n):
    """src, dst: host uint16 numpy arrays (F16 bits in, BF16 bits out)."""
    return _lib.rld_f16_to_bf16_host(src.ctypes.data, dst.ctypes.data, n)


def rld_lora_workspace_bytes(m, k_in, max_rank):
    return _lib.rld_lora_workspace_bytes(m, k_in, max_rank)


def rld_lora_shrink(pair, x, x_row_stride, m, xa, workspace, workspace_bytes, stream=None):
    return _lib.rld_lora_shrink(ctypes.byref(pair), ptr(x), x_row_stride, m, ptr(xa),
                                ptr(workspace), workspace_bytes, stream_handle(stream))


def rld_lora_expand_fold(pair, xa, m, base_out, out_row_stride, stream=None):
    return _lib.rld_lora_expand_fold(ctypes.byref(pair), ptr(xa), m, ptr(base_out),
                                     out_row_stride, stream_handle(stream))


def rld_lora_delta(pair, x, x_row_stride, m, base_out, out_row_stride, xa, workspace,
                   workspace_bytes, stream=None):
    return _lib.rld_lora_delta(ctypes.byref(pair), ptr(x), x_row_stride, m, ptr(base_out),
                               out_row_stride, ptr(xa), ptr(workspace), workspace_bytes,
                               stream_handle(stream))


def rld_moe_gather_shrink(route, x, x_row_stride, indices, row_adapter, top_k, n_rows, xa,
                          stream=None):
    return _lib.rld_moe_gather_shrink(ctypes.byref(route), ptr(x), x_row_stride, ptr(indices),
                                      ptr(row_adapter), top_k, n_rows, ptr(xa),
                                      stream_handle(stream))


def rld_moe_gather_expand_fold(route, xa, indices, row_adapter, top_k, n_rows, base_out,
                               out_row_stride, stream=None):
    return _lib.rld_moe_gather_expand_fold(ctypes.byref(route), ptr(xa), ptr(indices),
                                           ptr(row_adapter), top_k, n_rows, ptr(base_out),
                                           out_row_stride, stream_handle(stream))


def rld_moe_gather(route, x, x_row_stride, indices, row_adapter, top_k, n_rows, base_out,
                   out_row_stride, xa, stream=None):
    return _lib.rld_moe_gather(ctypes.byref(route), ptr(x), x_row_stride, ptr(indices),
                               ptr(row_adapter), top_k, n_rows, ptr(base_out), out_row_stride,
                               ptr(xa), stream_handle(stream))


def rld_moe_grouped_workspace_bytes(window_rows, k_in, max_rank, max_loras, num_experts):
    return _lib.rld_moe_grouped_workspace_bytes(window_rows, k_in, max_rank, max_loras,
                                                num_experts)


def rld_moe_grouped_shrink(route, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                           num_experts_off, sorted_token_ids, row_adapter, row_offset, row_end,
                           xa, xa_rows_cap, workspace, workspace_bytes, stream=None):
    return _lib.rld_moe_grouped_shrink(ctypes.byref(route), ptr(x), x_row_stride, int(x_gather),
                                       num_tokens, ptr(expert_offsets), num_experts_off,
                                       ptr(sorted_token_ids), ptr(row_adapter), row_offset,
                                       row_end, ptr(xa), xa_rows_cap, ptr(workspace),
                                       workspace_bytes, stream_handle(stream))


def rld_moe_grouped_expand_fold(route, xa, num_tokens, expert_offsets, num_experts_off,
                                sorted_token_ids, row_adapter, row_offset, row_end, base_out,
                                out_row_stride, stream=None):
    return _lib.rld_moe_grouped_expand_fold(ctypes.byref(route), ptr(xa), num_tokens,
                                            ptr(expert_offsets), num_experts_off,
                                            ptr(sorted_token_ids), ptr(row_adapter), row_offset,
                                            row_end, ptr(base_out), out_row_stride,
                                            stream_handle(stream))


def rld_moe_grouped(route, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                    num_experts_off, sorted_token_ids, row_adapter, row_offset, row_end, base_out,
                    out_row_stride, xa, xa_rows_cap, workspace, workspace_bytes, stream=None):
    return _lib.rld_moe_grouped(ctypes.byref(route), ptr(x), x_row_stride, int(x_gather),
                                num_tokens, ptr(expert_offsets), num_experts_off,
                                ptr(sorted_token_ids), ptr(row_adapter), row_offset, row_end,
                                ptr(base_out), out_row_stride, ptr(xa), xa_rows_cap,
                                ptr(workspace), workspace_bytes, stream_handle(stream))


def rld_moe_grouped_pair(route_a, route_b, x, x_row_stride, x_gather, num_tokens,
                         expert_offsets, num_experts_off, sorted_token_ids, row_adapter,
                         row_offset, row_end, base_a, os_a, base_b, os_b, xa_a, xa_b,
                         xa_rows_cap, workspace, workspace_bytes, stream=None):
    return _lib.rld_moe_grouped_pair(ctypes.byref(route_a), ctypes.byref(route_b), ptr(x),
                                     x_row_stride, int(x_gather), num_tokens,
                                     ptr(expert_offsets), num_experts_off,
                                     ptr(sorted_token_ids), ptr(row_adapter), row_offset,
                                     row_end, ptr(base_a), os_a, ptr(base_b), os_b, ptr(xa_a),
                                     ptr(xa_b), xa_rows_cap, ptr(workspace), workspace_bytes,
                                     stream_handle(stream))


def library_path() -> str:
    return LIB_PATH
