"""Plant plausible mistakes in a private copy of the oracle (CPU only) and check
that at least one pin of tests/test_oracle.py fails for each."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import test_oracle as T

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "rld_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("rld_oracle_mutant", ORACLE_SRC)
    m = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = m
    spec.loader.exec_module(m)
    return m


def _mut_truncating_round(m):
    orig = m.round_bf16

    def rb(v):
        v = np.asarray(v, np.float64)
        bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return np.where(np.isnan(v), orig(v), bits).astype(np.uint16)
    m.round_bf16 = rb


def _mut_fused_fold(m):
    def fold_row(x, w, out):
        xa = m.round_bf16(w.a64() @ m.bf16_to_f64(x))
        d = m.round_bf16(w.b64() @ m.bf16_to_f64(xa))
        s = m.bf16_to_f64(out) + np.float64(w.scale) * m.bf16_to_f64(d)
        return xa, m.round_bf16(s)
    m.fold_row = fold_row


def _mut_transposed_A(m):
    def fold_row(x, w, out):
        xa = m.round_bf16(m.bf16_to_f64(x) @ w.a64())
        d = m.round_bf16(w.b64() @ m.bf16_to_f64(xa))
        t = np.float32(w.scale) * m.bf16_to_f32(d)
        return xa, m.round_bf16(m.bf16_to_f32(out) + t)
    m.fold_row = fold_row


def _mut_dropped_term(m):
    def fold_row(x, w, out):
        xa = m.round_bf16(w.a64()[:, :-1] @ m.bf16_to_f64(x)[:-1])
        d = m.round_bf16(w.b64() @ m.bf16_to_f64(xa))
        t = np.float32(w.scale) * m.bf16_to_f32(d)
        return xa, m.round_bf16(m.bf16_to_f32(out) + t)
    m.fold_row = fold_row


def _mut_scale_before_round(m):
    def fold_row(x, w, out):
        xa = m.round_bf16(w.a64() @ m.bf16_to_f64(x))
        d = m.round_bf16(np.float64(w.scale) * (w.b64() @ m.bf16_to_f64(xa)))
        return xa, m.round_bf16(m.bf16_to_f32(out) + m.bf16_to_f32(d))
    m.fold_row = fold_row


def _mut_unrounded_xa(m):
    def fold_row(x, w, out):
        xa_exact = w.a64() @ m.bf16_to_f64(x)
        d = m.round_bf16(w.b64() @ xa_exact)
        t = np.float32(w.scale) * m.bf16_to_f32(d)
        return m.round_bf16(xa_exact), m.round_bf16(m.bf16_to_f32(out) + t)
    m.fold_row = fold_row


def _mut_sign(m):
    def fold_row(x, w, out):
        xa = m.round_bf16(w.a64() @ m.bf16_to_f64(x))
        d = m.round_bf16(w.b64() @ m.bf16_to_f64(xa))
        t = np.float32(w.scale) * m.bf16_to_f32(d)
        return xa, m.round_bf16(m.bf16_to_f32(out) - t)
    m.fold_row = fold_row


def _mut_rslora_always(m):
    import math
    m.scale_for = lambda alpha, rank, rs: np.float32(alpha / math.sqrt(rank))


def _mut_gather_token_mod(m):
    m.gather_row_token = lambda row, top_k: row % top_k


def _mut_owner_off_by_one(m):
    def expert_owner(off, lo, hi):
        off = np.asarray(off, np.int64)
        owner = np.full(hi - lo, -1, np.int64)
        for e in range(len(off) - 1):
            a, b = max(int(off[e]) + 1, lo), min(int(off[e + 1]) + 1, hi)
            if a < b:
                owner[a - lo:b - lo] = e
        return owner
    m.expert_owner = expert_owner


def _mut_grouped_adapter_by_row(m):
    orig = m.moe_grouped

    def moe_grouped(pairs, E, k_in, n_out, R, x, xs, xg, nt, off, stid, ra, lo, hi, base, os_):
        # looks the adapter up with the sorted row index instead of the token
        fake = None if ra is None else np.resize(ra, max(len(stid), 1))
        return orig(pairs, E, k_in, n_out, R, x, xs, xg, len(stid) if stid is not None else nt,
                    off, None if stid is None else np.arange(len(stid), dtype=np.int32) if not xg
                    else stid, fake, lo, hi, base, os_)
    m.moe_grouped = moe_grouped


def _mut_ignore_out_offset(m):
    orig = m.bgmv
    m.bgmv = lambda s, k, n_out, R, x, xs, seq, n, base, off, os_: orig(
        s, k, n_out, R, x, xs, seq, n, base, 0, os_)


def _mut_xa_not_zeroed(m):
    orig = m.bgmv

    def bgmv(*a):
        xa, out = orig(*a)
        seq = a[6]
        xa[np.asarray(seq[:len(xa)]) < 0] = 0x3F80
        return xa, out
    m.bgmv = bgmv


def _mut_wc_floor(m):
    m.grouped_down_wc = lambda lo, hi: max(1, (hi - lo) // 64)


def _mut_pack_first_wins(m):
    orig = m.pack_expert_tables

    def pet(entries):
        return orig(list(reversed(entries)))
    m.pack_expert_tables = pet


def _lora_variant(m, *, b_orient="ok", fused=False, round_xa=True, x_stride_ok=True):
    """A re-implementation of the matrix-form unrouted delta with one mistake."""
    def lora_delta(w, k_in, n_out, max_rank, x, xs, rows, base, off, os_):
        out = np.array(base, dtype=np.uint16, copy=True)
        if rows == 0:
            return np.zeros((0, max_rank), np.uint16), out
        st = xs if x_stride_ok else k_in
        X = m.bf16_to_f64(np.asarray(x)[np.arange(rows)[:, None] * st + np.arange(k_in)])
        XA64 = X @ w.a64().T
        XA = m.round_bf16(XA64)
        Bm = w.b64() if b_orient == "ok" else w.b64().reshape(max_rank, n_out).T
        D64 = (m.bf16_to_f64(XA) if round_xa else XA64) @ Bm.T
        D = m.round_bf16(D64)
        ro = off + np.arange(rows)[:, None] * os_ + np.arange(n_out)
        if fused:
            S = m.bf16_to_f64(out[ro]) + np.float64(w.scale) * m.bf16_to_f64(D)
        else:
            S = m.bf16_to_f32(out[ro]) + np.float32(w.scale) * m.bf16_to_f32(D)
        out[ro] = m.round_bf16(S)
        return XA, out
    m.lora_delta = lora_delta


def _mut_lora_transposed_B(m):
    _lora_variant(m, b_orient="transposed")


def _mut_lora_fused_fold(m):
    _lora_variant(m, fused=True)


def _mut_lora_unrounded_xa(m):
    _lora_variant(m, round_xa=False)


def _mut_lora_ignores_x_stride(m):
    _lora_variant(m, x_stride_ok=False)


def _grouped_variant(m, *, token_rule="given", expert_rule="skip"):
    """A re-implementation of the grouped window fold with one mistake in the
    rules for values the host cannot check."""
    def moe_grouped(pairs, E, k_in, n_out, R, x, xs, xg, nt, off, stid, ra, lo, hi, base, os_):
        xa = np.zeros((max(hi - lo, 0), R), np.uint16)
        out = np.array(base, dtype=np.uint16, copy=True)
        if hi <= lo:
            return xa, out
        owner = m.expert_owner(off, lo, hi)
        if token_rule == "given":
            need = stid is not None
        elif token_rule == "gather_or_adapter":  # tokens of down rows never checked
            need = xg or ra is not None
        else:  # "never": no range check at all
            need = False
        for r in range(lo, hi):
            e = int(owner[r - lo])
            if e < 0:
                continue
            if e >= E:
                if expert_rule == "skip":
                    continue
                if expert_rule == "clamp":
                    e = E - 1
            t = int(stid[r]) if stid is not None else -1
            if need and not (0 <= t < nt):
                continue
            s = int(ra[t]) if ra is not None else 0
            if not (0 <= s < len(pairs)):
                continue
            w = pairs[s][e]
            if w is None or not w.active:
                continue
            xr = t if xg else r
            o0 = r * os_
            xa[r - lo], out[o0:o0 + n_out] = m.fold_row(x[xr * xs: xr * xs + k_in], w,
                                                        out[o0:o0 + n_out])
        return xa, out
    m.moe_grouped = moe_grouped


def _mut_grouped_tokens_unchecked(m):
    _grouped_variant(m, token_rule="never")


def _mut_grouped_tokens_checked_only_when_used(m):
    _grouped_variant(m, token_rule="gather_or_adapter")


def _mut_grouped_expert_past_table_clamped(m):
    _grouped_variant(m, expert_rule="clamp")


def _mut_grouped_expert_past_table_unchecked(m):
    _grouped_variant(m, expert_rule="none")


MUTANTS = [_mut_truncating_round, _mut_fused_fold, _mut_transposed_A, _mut_dropped_term,
           _mut_scale_before_round, _mut_unrounded_xa, _mut_sign, _mut_rslora_always,
           _mut_gather_token_mod, _mut_owner_off_by_one, _mut_grouped_adapter_by_row,
           _mut_ignore_out_offset, _mut_xa_not_zeroed, _mut_wc_floor, _mut_pack_first_wins,
           _mut_lora_transposed_B, _mut_lora_fused_fold, _mut_lora_unrounded_xa,
           _mut_lora_ignores_x_stride, _mut_grouped_tokens_unchecked,
           _mut_grouped_tokens_checked_only_when_used, _mut_grouped_expert_past_table_clamped,
           _mut_grouped_expert_past_table_unchecked]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__)
def test_a_pin_catches(mutate):
    m = fresh_oracle()
    mutate(m)
    failed = []
    for pin in T.PINS:
        try:
            pin(m)
        except Exception:  # an assertion or a shape error both count as caught
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutate.__name__}"
