"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin is a function taking the oracle module, so the mutation tests at the
end can plant a mistake in a copy of the oracle (on the CPU) and check that a
pin catches it.  No GPU is used here.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

# ---------------------------------------------------------------------------
# exact-rational reference for brute force (independent of the oracle's floats)
# ---------------------------------------------------------------------------


def _round_frac(q: Fraction, p: int, emin: int, emax: int):
    """Round a rational to a binary format with p significant bits, ties to even.
    Returns a Fraction, or +-inf as float."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    big = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > big:
        return sign * math.inf
    return sign * r


def _to_bf16_bits_frac(q):
    r = _round_frac(q, 8, -126, 127)
    f = float(r)
    return int((np.array([f], np.float32).view(np.uint32)[0] >> 16))


def _to_f32_frac(q):
    return Fraction(float(np.float32(float(_round_frac(q, 24, -126, 127)))))


def _bf(bits):
    return Fraction(float(O.bf16_to_f64(np.array([bits], np.uint16))[0]))


def exact_fold_row(x_bits, A_bits, B_bits, scale_f32, out_bits):
    """The fold of one row in exact rationals, rounding only where the pages do."""
    R, K = A_bits.shape
    xa = []
    for k in range(R):
        acc = sum((_bf(x_bits[c]) * _bf(A_bits[k, c]) for c in range(K)), Fraction(0))
        xa.append(_to_bf16_bits_frac(acc))
    outs = []
    for j in range(B_bits.shape[0]):
        acc = sum((_bf(xa[k]) * _bf(B_bits[j, k]) for k in range(R)), Fraction(0))
        d = _bf(_to_bf16_bits_frac(acc))
        t = _to_f32_frac(Fraction(float(scale_f32)) * d)
        s = _to_f32_frac(_bf(out_bits[j]) + t)
        outs.append(_to_bf16_bits_frac(s))
    return np.array(xa, np.uint16), np.array(outs, np.uint16)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

# hand-derived BF16 bit patterns (value, bits)
BF16_KNOWN = [
    (1.0, 0x3F80),
    (-2.0, 0xC000),
    (1.0 + 2.0 ** -8, 0x3F80),            # tie between 0x3F80 and 0x3F81 -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 0x3F81 and 0x3F82 -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie
    (0.1, 0x3DCD),
    (1.0 / 3.0, 0x3EAB),
    ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
    ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie above the largest finite -> inf
    ((2.0 - 2.0 ** -8 - 2.0 ** -30) * 2.0 ** 127, 0x7F7F),
    (2.0 ** -133, 0x0001),                # smallest subnormal
    (2.0 ** -134, 0x0000),                # tie with zero -> even (zero)
    (3 * 2.0 ** -134, 0x0002),            # tie between 1 and 2 units -> even
    (2.0 ** -126, 0x0080),                # smallest normal
    (2.0 ** -126 - 2.0 ** -134, 0x0080),  # tie between 0x007F and 0x0080 -> even
    (-0.0, 0x8000),
    (math.inf, 0x7F80),
    (-math.inf, 0xFF80),
]


def pin_bf16_known(o):
    vals = np.array([v for v, _ in BF16_KNOWN], np.float64)
    got = o.round_bf16(vals)
    want = np.array([b for _, b in BF16_KNOWN], np.uint16)
    assert np.array_equal(got, want), [hex(g) for g in got]
    nan = o.round_bf16(np.array([math.nan, -math.nan]))
    assert nan[0] == 0x7FC0 and nan[1] == 0xFFC0


def pin_bf16_roundtrip(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = o.bf16_to_f64(bits)
    got = o.round_bf16(v)
    finite = np.isfinite(v)
    assert np.array_equal(got[finite], bits[finite])
    isnan = np.isnan(v)
    assert np.all((got[isnan] & 0x7FC0) == 0x7FC0)


def pin_bf16_midpoints(o):
    # midpoint between consecutive positive finite BF16 values b and b+1, built
    # from the integer bit patterns; ties go to the even pattern.
    rng = np.random.default_rng(5)
    b = rng.integers(0x0001, 0x7F7F, size=20000).astype(np.uint16)
    lo = o.bf16_to_f64(b)
    hi = o.bf16_to_f64(b + 1)
    mid = (lo + hi) / 2.0  # exact in float64
    got = o.round_bf16(mid)
    want = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # a hair off the midpoint goes to the nearer value
    below = np.nextafter(mid, 0.0)
    assert np.array_equal(o.round_bf16(below), b)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(o.round_bf16(above), (b + 1).astype(np.uint16))


def pin_bf16_vs_torch(o):
    # float32 -> bfloat16 in torch rounds to nearest even: a library special case
    rng = np.random.default_rng(6)
    with np.errstate(over="ignore"):
        f = _f32_samples(rng)
    f = f[np.isfinite(f)]
    t = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.round_bf16(f.astype(np.float64))
    assert np.array_equal(got, t)


def _f32_samples(rng):
    return np.concatenate([
        rng.standard_normal(50000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),
        (rng.standard_normal(20000) * 1e38).astype(np.float32),
        rng.integers(0, 2 ** 32, size=50000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])


def pin_scale_closed_forms(o):
    f32bits = lambda v: int(np.array([v], np.float32).view(np.uint32)[0])  # noqa: E731
    assert f32bits(o.scale_for(16.0, 8, False)) == 0x40000000   # 2
    assert f32bits(o.scale_for(16.0, 4, False)) == 0x40800000   # 4
    assert f32bits(o.scale_for(32.0, 64, False)) == 0x3F000000  # 0.5
    assert f32bits(o.scale_for(32.0, 64, True)) == 0x40800000   # 32/8 = 4
    assert f32bits(o.scale_for(32.0, 16, True)) == 0x41000000   # 32/4 = 8
    assert f32bits(o.scale_for(32.0, 8, True)) == 0x413504F3    # 8*sqrt(2)
    assert f32bits(o.scale_for(32.0, 32, True)) == 0x40B504F3   # 4*sqrt(2)
    assert o.scale_for(7.0, 1, True) == o.scale_for(7.0, 1, False) == np.float32(7.0)


def _tiny_slots(o, rng, k_in, n_out, max_rank, ranks):
    ads = [W.make_adapter(rng, s, r, k_in, n_out, 16.0, s % 2 == 1) for s, r in enumerate(ranks)]
    return ads, o.pack_slots(ads, len(ranks), max_rank)


def pin_brute_force_bgmv(o):
    rng = W.rng_for(0, salt=11)
    k_in, n_out, max_rank = 24, 16, 8
    ads, slots = _tiny_slots(o, rng, k_in, n_out, max_rank, [5, 8])
    n = 4
    seq = np.array([1, 0, -1, 1], np.int32)
    x = W.bf16_trunc(rng.standard_normal((n, k_in)).astype(np.float32)).ravel()
    base = W.bf16_trunc(rng.standard_normal((n, n_out)).astype(np.float32)).ravel()
    xa, out = o.bgmv(slots, k_in, n_out, max_rank, x, k_in, seq, n, base, 0, n_out)
    for i in range(n):
        s = int(seq[i])
        if s < 0:
            assert np.all(xa[i] == 0)
            assert np.array_equal(out[i * n_out:(i + 1) * n_out], base[i * n_out:(i + 1) * n_out])
            continue
        ad = ads[s]
        Ap, Bp = np.zeros((max_rank, k_in), np.uint16), np.zeros((n_out, max_rank), np.uint16)
        Ap[:ad.rank] = ad.A
        Bp[:, :ad.rank] = ad.B
        sc = np.float32(ad.alpha / math.sqrt(ad.rank) if ad.use_rslora else ad.alpha / ad.rank)
        exa, eout = exact_fold_row(x[i * k_in:(i + 1) * k_in], Ap, Bp, sc,
                                   base[i * n_out:(i + 1) * n_out])
        assert np.array_equal(xa[i], exa)
        assert np.array_equal(out[i * n_out:(i + 1) * n_out], eout)


def _int_bits(a):
    """small integers -> BF16 bits (exact: |a| <= 256)."""
    return O.round_bf16(np.asarray(a, np.float64))


def pin_textbook_lora(o):
    """max_loras=1, every row on slot 0, integer-exact values: the fold must equal
    standard LoRA  y = W0 x + (alpha/r) B (A x)  with A [r, k_in], B [n_out, r]."""
    rng = np.random.default_rng(9)
    for k_in, n_out, rank, max_rank in ((8, 8, 8, 8), (16, 12, 4, 8), (12, 20, 3, 8)):
        n = 5
        x = rng.integers(-1, 2, size=(n, k_in))
        A = rng.integers(-1, 2, size=(rank, k_in))
        B = rng.integers(-1, 2, size=(n_out, rank))
        base = 2 * rng.integers(-4, 5, size=(n, n_out))
        alpha = 2.0 * rank  # scale 2
        ad = W.Adapter(0, rank, alpha, False, _int_bits(A), _int_bits(B))
        slots = o.pack_slots([ad], 1, max_rank)
        xa, out = o.bgmv(slots, k_in, n_out, max_rank, _int_bits(x).ravel(), k_in,
                         np.zeros(n, np.int32), n, _int_bits(base).ravel(), 0, n_out)
        y = base + 2 * (x @ A.T) @ B.T  # textbook, exact integers
        assert np.array_equal(o.bf16_to_f64(out).reshape(n, n_out), y.astype(np.float64))
        assert np.array_equal(o.bf16_to_f64(xa)[:, :rank], (x @ A.T).astype(np.float64))


def pin_pad_invariant(o):
    rng = W.rng_for(0, salt=12)
    k_in, n_out = 40, 24
    ads = [W.make_adapter(rng, 0, 5, k_in, n_out, 16.0, False),
           W.make_adapter(rng, 1, 3, k_in, n_out, 16.0, True)]
    n = 6
    seq = np.array([0, 1, 1, -1, 0, 1], np.int32)
    x = W.bf16_trunc(rng.standard_normal((n, k_in)).astype(np.float32)).ravel()
    base = W.bf16_trunc(rng.standard_normal((n, n_out)).astype(np.float32)).ravel()
    xa16, out16 = o.bgmv(o.pack_slots(ads, 2, 16), k_in, n_out, 16, x, k_in, seq, n, base, 0, n_out)
    for s, ad in enumerate(ads):
        # the same slot alone at its true rank
        only = [None, None]
        only[s] = o.pack_slots([ad], 2, ad.rank)[s]
        xa_t, out_t = o.bgmv(only, k_in, n_out, ad.rank, x, k_in, seq, n, base, 0, n_out)
        rows = np.where(seq == s)[0]
        assert np.array_equal(xa16[rows, :ad.rank], xa_t[rows])
        assert np.all(xa16[rows, ad.rank:] == 0)
        for i in rows:
            assert np.array_equal(out16[i * n_out:(i + 1) * n_out], out_t[i * n_out:(i + 1) * n_out])


def pin_inactive_and_strides(o):
    """Base rows (slot <0, slot >= max_loras, missing A or B) and everything outside
    [0,n_out) of each row stay bit-identical; K folds inside [Q|K|V] rows."""
    rng = W.rng_for(0, salt=13)
    k_in, n_out, max_rank, max_loras = 32, 16, 8, 4
    ads = [W.make_adapter(rng, s, 8, k_in, n_out, 16.0, False) for s in range(max_loras)]
    slots = o.pack_slots(ads, max_loras, max_rank)
    slots[2] = o.SlotWeights(slots[2].A, None, slots[2].scale)  # b_table entry 0
    slots[3] = o.SlotWeights(None, slots[3].B, slots[3].scale)  # a_table entry 0
    seq = np.array([0, -1, 4, 7, 2, 3, 1, -5], np.int32)
    n = len(seq)
    xs, os_, off = k_in + 8, 3 * n_out, n_out  # x padded rows; out rows [Q|K|V], K region
    x = W.bf16_trunc(rng.standard_normal(n * xs).astype(np.float32))
    base = W.bf16_trunc(rng.standard_normal(n * os_).astype(np.float32))
    xa, out = o.bgmv(slots, k_in, n_out, max_rank, x, xs, seq, n, base, off, os_)
    changed = out != base
    mask = np.zeros(n * os_, bool)
    for i in range(n):
        if seq[i] in (0, 1):
            mask[i * os_ + off: i * os_ + off + n_out] = True
    assert not np.any(changed & ~mask)
    assert np.any(changed)
    for i in range(n):
        if seq[i] not in (0, 1):
            assert np.all(xa[i] == 0)


def pin_batched_equals_rows(o):
    rng = W.rng_for(0, salt=14)
    k_in, n_out, max_rank = 48, 32, 8
    ads, slots = _tiny_slots(o, rng, k_in, n_out, max_rank, [8, 6, 4])
    n = 7
    seq = rng.integers(-1, 3, size=n).astype(np.int32)
    x = W.bf16_trunc(rng.standard_normal(n * k_in).astype(np.float32))
    base = W.bf16_trunc(rng.standard_normal(n * n_out).astype(np.float32))
    xa, out = o.bgmv(slots, k_in, n_out, max_rank, x, k_in, seq, n, base, 0, n_out)
    for i in range(n):
        xa1, out1 = o.bgmv(slots, k_in, n_out, max_rank, x[i * k_in:(i + 1) * k_in], k_in,
                           seq[i:i + 1], 1, base[i * n_out:(i + 1) * n_out], 0, n_out)
        assert np.array_equal(xa[i], xa1[0])
        assert np.array_equal(out[i * n_out:(i + 1) * n_out], out1)


def pin_fold_order(o):
    """scale*delta is rounded to fp32 before the add (base += scale*bf16(delta)):
    scale = 1+2^-23, delta = 1+2^-7, base = -(1+2^-7) gives exactly 2^-23
    (BF16 0x3400); a fused multiply-add would keep 2^-23+2^-30 (0x3401)."""
    scale = np.float32(1.0 + 2.0 ** -23)
    d = np.uint16(0x3F81)
    base = np.uint16(0xBF81)
    # one-row, rank-1, k_in=1 problem whose delta is exactly d: x = 1, A = 1, B = d
    w = o.SlotWeights(np.array([[0x3F80]], np.uint16), np.array([[d]], np.uint16), scale)
    xa, out = o.fold_row(np.array([0x3F80], np.uint16), w, np.array([base], np.uint16))
    assert xa[0] == 0x3F80
    assert out[0] == 0x3400


def _probe_grouped_workload(num_tokens=300, top_k=4, num_experts=16, max_loras=3,
                            k_in=16, n_out=8, rank=4, max_rank=8, seed=21):
    """Routing probe: x rows carry (1, token_hi, token_lo); A_{s,e} selects them;
    B_{s,e} writes (e, s, token_hi, token_lo, 1).  scale 1, base 0, so a folded row
    reads back its expert, slot and token exactly."""
    rng = np.random.default_rng(seed)
    topk = W.route_topk(rng, num_tokens, num_experts, top_k)
    offsets, stid, sexp, _ = W.expert_sort(topk, num_experts)
    te = num_tokens * top_k
    row_adapter = rng.integers(-1, max_loras, size=num_tokens).astype(np.int32)
    adapted = rng.random((max_loras, num_experts)) < 0.6

    def xrow_for(t):
        v = np.zeros(k_in)
        v[0], v[1], v[2] = 1, t // 64, t % 64
        v[3:] = rng.integers(-3, 4, size=k_in - 3)  # ignored by A
        return v

    adapters = []
    for s in range(max_loras):
        for e in range(num_experts):
            if not adapted[s, e]:
                continue
            A = np.zeros((rank, k_in))
            A[0, 0] = A[1, 1] = A[2, 2] = 1
            B = np.zeros((n_out, rank))
            B[0, 0], B[1, 0], B[2, 1], B[3, 2], B[4, 0] = e, s, 1, 1, 1
            adapters.append(W.Adapter(s, rank, float(rank), False, _int_bits(A), _int_bits(B), e))
    x_tok = _int_bits(np.stack([xrow_for(t) for t in range(num_tokens)]))
    x_sorted = _int_bits(np.stack([xrow_for(int(t)) for t in stid]))
    return dict(num_tokens=num_tokens, top_k=top_k, num_experts=num_experts, te=te,
                offsets=offsets, stid=stid, sexp=sexp, row_adapter=row_adapter,
                adapted=adapted, adapters=adapters, x_tok=x_tok, x_sorted=x_sorted,
                k_in=k_in, n_out=n_out, max_rank=max_rank, max_loras=max_loras, rank=rank)


def pin_routing_probe_grouped(o):
    P = _probe_grouped_workload()
    pairs = o.pack_expert_pairs(P["adapters"], P["max_loras"], P["num_experts"], P["max_rank"])
    te, n_out = P["te"], P["n_out"]
    base = np.zeros(te * n_out, np.uint16)
    for gather in (False, True):
        for ra in (P["row_adapter"], None):
            x = P["x_tok"] if gather else P["x_sorted"]
            lo, hi = 37, te - 11  # a window that cuts through expert spans
            xa, out = o.moe_grouped(pairs, P["num_experts"], P["k_in"], n_out, P["max_rank"],
                                    x.ravel(), P["k_in"], gather, P["num_tokens"], P["offsets"],
                                    P["stid"], ra, lo, hi, base, n_out)
            out = o.bf16_to_f64(out).reshape(te, n_out)
            xa = o.bf16_to_f64(xa)
            for r in range(te):
                t, e = int(P["stid"][r]), int(P["sexp"][r])
                s = int(ra[t]) if ra is not None else 0
                folds = lo <= r < hi and s >= 0 and P["adapted"][s, e]
                want = np.zeros(n_out)
                if folds:
                    want[:5] = (e, s, t // 64, t % 64, 1)
                assert np.array_equal(out[r], want), (gather, r)
                if lo <= r < hi:
                    wxa = np.zeros(P["max_rank"])
                    if folds:
                        wxa[:3] = (1, t // 64, t % 64)
                    assert np.array_equal(xa[r - lo], wxa)


def pin_grouped_invalid_values(o):
    """Grouped-path values the host cannot check ("Module moe_lora_grouped",
    moe_lora_grouped_down: per-tile early return on empty, out-of-range or
    unadapted expert spans), on the closed-form routing probe:
      * sorted_token_ids entries >= num_tokens or < 0: whenever the map is
        given, such a row is a base row, in all four combinations of x gather
        and row_adapter; without the map (no gather, no row_adapter) no token
        is read and every row of an adapted span folds on slot 0;
      * an offsets array that lists more experts than the table holds: rows of
        the experts past the table are base rows.
    The base is -0.0 everywhere, so an untouched row (-0.0 bits) differs from a
    row folded with a zero delta (-0.0 + 0 = +0.0)."""
    P = _probe_grouped_workload()
    te, n_out, R_ = P["te"], P["n_out"], P["max_rank"]
    E_tab = P["num_experts"] - 4  # table of experts 0..11; offsets list 16
    ads = [a for a in P["adapters"] if a.expert < E_tab]
    pairs = o.pack_expert_pairs(ads, P["max_loras"], E_tab, R_)
    stid = P["stid"].copy()
    bad_rows = {3: P["num_tokens"], 58: 10 ** 6, 131: -1, 402: -7, te - 20: P["num_tokens"] + 3}
    for r, t in bad_rows.items():
        stid[r] = t
    base = np.full(te * n_out, 0x8000, np.uint16)
    neg0 = np.uint16(0x8000)
    lo, hi = 2, te - 5
    for gather in (False, True):
        for ra in (P["row_adapter"], None):
            for map_given in ((True, False) if (not gather and ra is None) else (True,)):
                x = P["x_tok"] if gather else P["x_sorted"]
                xa, out = o.moe_grouped(pairs, E_tab, P["k_in"], n_out, R_, x.ravel(), P["k_in"],
                                        gather, P["num_tokens"], P["offsets"],
                                        stid if map_given else None, ra, lo, hi, base, n_out)
                out = out.reshape(te, n_out)
                for r in range(te):
                    e, t = int(P["sexp"][r]), int(stid[r])
                    tok_ok = (0 <= t < P["num_tokens"]) or not map_given
                    s = int(ra[t]) if (ra is not None and tok_ok) else 0
                    folds = (lo <= r < hi and e < E_tab and tok_ok and s >= 0
                             and bool(P["adapted"][s, e]))
                    tx = t if gather else int(P["stid"][r])  # token whose x row is read
                    if folds:
                        want = np.zeros(n_out)
                        want[:5] = (e, s, tx // 64, tx % 64, 1)
                        assert np.array_equal(out[r], o.round_bf16(want)), (gather, r)
                    else:
                        assert np.all(out[r] == neg0), (gather, ra is None, map_given, r)
                    if lo <= r < hi:
                        wxa = np.zeros(R_)
                        if folds:
                            wxa[:3] = (1, tx // 64, tx % 64)
                        assert np.array_equal(xa[r - lo], o.round_bf16(wxa)), (gather, r)
                if map_given:
                    assert all(np.all(out[r] == neg0) for r in bad_rows)


def pin_routing_probe_gather(o):
    P = _probe_grouped_workload(num_tokens=40, top_k=8, num_experts=32, max_loras=4, seed=22)
    pairs = o.pack_expert_pairs(P["adapters"], P["max_loras"], P["num_experts"], P["max_rank"])
    rng = np.random.default_rng(23)
    T, K = P["num_tokens"], P["top_k"]
    indices = np.stack([rng.choice(P["num_experts"], size=K, replace=False)
                        for _ in range(T)]).astype(np.int32).ravel()
    indices[5] = -1          # invalid expert ids are skipped
    indices[9] = P["num_experts"]
    row_tok = []  # token of each flat row, by construction (token-major rows)
    xr = []
    for t in range(T):
        for _ in range(K):
            row_tok.append(t)
            v = np.zeros(P["k_in"])
            rho = len(xr)
            v[0], v[1], v[2] = 1, rho // 64, rho % 64
            xr.append(v)
    x = _int_bits(np.stack(xr))
    n_rows, n_out = T * K, P["n_out"]
    base = np.zeros(n_rows * n_out, np.uint16)
    for ra in (P["row_adapter"], None):
        xa, out = o.moe_gather(pairs, P["num_experts"], P["k_in"], n_out, P["max_rank"],
                               x.ravel(), P["k_in"], indices, ra, K, n_rows, base, n_out)
        out = o.bf16_to_f64(out).reshape(n_rows, n_out)
        for rho in range(n_rows):
            e, t = int(indices[rho]), row_tok[rho]
            s = int(ra[t]) if ra is not None else 0
            folds = 0 <= e < P["num_experts"] and s >= 0 and P["adapted"][s, e]
            want = np.zeros(n_out)
            if folds:
                want[:5] = (e, s, rho // 64, rho % 64, 1)
            assert np.array_equal(out[rho], want), rho


def _small_grouped(o, seed=4, num_tokens=200, projections=("down", "gate")):
    wl = W.moe_grouped(seed, num_tokens=num_tokens, top_k=4, num_experts=16, hidden=64,
                       inter=48, max_loras=3, n_adapted=12, ranks=(4, 8), max_rank=8,
                       cap=256, projections=projections)
    return wl


def pin_window_union(o):
    wl = _small_grouped(o)
    for p in wl.projections:
        pairs = o.pack_expert_pairs(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank)
        args = (pairs, wl.num_experts, p.k_in, p.n_out, wl.max_rank, p.x.ravel(), p.k_in,
                p.x_gather, wl.num_tokens, wl.expert_offsets, wl.sorted_token_ids,
                wl.row_adapter)
        xa_full, out_full = o.moe_grouped(*args, 0, wl.te, p.base.ravel(), p.n_out)
        for cap in (64, 100, 333, wl.te + 5):
            out = p.base.ravel().copy()
            xas = []
            for lo, hi in o.grouped_down_windows(wl.te, cap):
                xa, out = o.moe_grouped(*args, lo, hi, out, p.n_out)
                xas.append(xa)
            assert np.array_equal(np.concatenate(xas), xa_full)
            assert np.array_equal(out, out_full)


def pin_cross_path(o):
    """A grouped (sorted) row, its unsorted gather row and a one-row BGMV with the
    same (A, B, scale) fold identically."""
    wl = _small_grouped(o, projections=("down",))
    p = wl.projections[0]
    pairs = o.pack_expert_pairs(p.adapters, wl.max_loras, wl.num_experts, wl.max_rank)
    xa_g, out_g = o.moe_grouped(pairs, wl.num_experts, p.k_in, p.n_out, wl.max_rank,
                                p.x.ravel(), p.k_in, False, wl.num_tokens, wl.expert_offsets,
                                wl.sorted_token_ids, wl.row_adapter, 0, wl.te,
                                p.base.ravel(), p.n_out)
    out_g = out_g.reshape(wl.te, p.n_out)
    n_checked = 0
    for r in range(0, wl.te, 7):
        t, e = int(wl.sorted_token_ids[r]), int(wl.sorted_expert[r])
        s = int(wl.row_adapter[t])
        if s < 0 or pairs[s][e] is None:
            continue
        xa1, out1 = o.bgmv([pairs[s][e]], p.k_in, p.n_out, wl.max_rank, p.x[r], p.k_in,
                           np.zeros(1, np.int32), 1, p.base[r], 0, p.n_out)
        assert np.array_equal(xa1[0], xa_g[r]) and np.array_equal(out1, out_g[r])
        # the same row presented unsorted to the gather path (one flat row, top_k=1)
        xa2, out2 = o.moe_gather(pairs, wl.num_experts, p.k_in, p.n_out, wl.max_rank, p.x[r],
                                 p.k_in, np.array([e], np.int32), np.array([s], np.int32), 1, 1,
                                 p.base[r], p.n_out)
        assert np.array_equal(xa2[0], xa_g[r]) and np.array_equal(out2, out_g[r])
        n_checked += 1
    assert n_checked > 5


def pin_helpers(o):
    # grouped_down_wc: ceil(len/64), min 1; a full window gives ceil(te/64)
    assert o.grouped_down_wc(0, 32768) == 512
    assert o.grouped_down_wc(0, 8192) == 128
    assert o.grouped_down_wc(8192, 8192) == 1
    assert o.grouped_down_wc(10, 75) == 2
    assert o.grouped_down_wc(0, 64) == 1 and o.grouped_down_wc(0, 65) == 2
    # windows: contiguous, cover 0..total, each at most cap
    for total, cap in ((32768, 8192), (1000, 333), (5, 8), (0, 4), (64, 64)):
        w = o.grouped_down_windows(total, cap)
        assert [a for a, _ in w] == [b for _, b in [(0, 0)] + w[:-1]] if w else total == 0
        if w:
            assert w[0][0] == 0 and w[-1][1] == total
            assert all(0 < b - a <= cap for a, b in w)
    assert o.grouped_down_windows(32768, 8192) == [(0, 8192), (8192, 16384), (16384, 24576),
                                                   (24576, 32768)]
    assert o.gather_row_token(0, 8) == 0 and o.gather_row_token(7, 8) == 0
    assert o.gather_row_token(8, 8) == 1 and o.gather_row_token(255, 8) == 31
    # pack_expert_tables: None when empty; n = max id + 1; zeros where unadapted; last wins
    assert o.pack_expert_tables([]) is None
    n, a, b, sc = o.pack_expert_tables([(3, 0x100, 0x200, 0.5), (1, 0x300, 0x400, 2.0),
                                        (3, 0x500, 0x600, 4.0)])
    assert n == 4
    assert a == [0, 0x300, 0, 0x500] and b == [0, 0x400, 0, 0x600]
    assert [float(v) for v in sc] == [0.0, 2.0, 0.0, 4.0]


def _one_pair(o, rng, k_in, n_out, rank, max_rank, rslora=False):
    ad = W.make_adapter(rng, 0, rank, k_in, n_out, 16.0, rslora)
    return ad, o.pack_slots([ad], 1, max_rank)[0]


def pin_lora_delta_brute_force(o):
    """Unrouted delta (apply_lora_delta) on tiny inputs against exact rationals,
    rounding only where the pages do; rank padded, rsLoRA scale."""
    rng = W.rng_for(0, salt=21)
    k_in, n_out, max_rank, m = 20, 12, 8, 3
    ad, w = _one_pair(o, rng, k_in, n_out, 5, max_rank, rslora=True)
    x = W.bf16_trunc(rng.standard_normal((m, k_in)).astype(np.float32)).ravel()
    base = W.bf16_trunc(rng.standard_normal((m, n_out)).astype(np.float32)).ravel()
    xa, out = o.lora_delta(w, k_in, n_out, max_rank, x, k_in, m, base, 0, n_out)
    for i in range(m):
        exa, eout = exact_fold_row(x[i * k_in:(i + 1) * k_in], w.A, w.B, w.scale,
                                   base[i * n_out:(i + 1) * n_out])
        assert np.array_equal(xa[i], exa)
        assert np.array_equal(out[i * n_out:(i + 1) * n_out], eout)


def pin_lora_delta_textbook(o):
    """Integer-exact values: the unrouted delta is standard LoRA
    y = W0 x + (alpha/r) B (A x), A [r, k_in], B [n_out, r]."""
    rng = np.random.default_rng(23)
    for k_in, n_out, rank, max_rank, m in ((8, 8, 8, 8, 1), (16, 12, 4, 8, 6), (12, 20, 3, 16, 9)):
        x = rng.integers(-1, 2, size=(m, k_in))
        A = rng.integers(-1, 2, size=(rank, k_in))
        B = rng.integers(-1, 2, size=(n_out, rank))
        base = 2 * rng.integers(-4, 5, size=(m, n_out))
        ad = W.Adapter(0, rank, 4.0 * rank, False, _int_bits(A), _int_bits(B))  # scale 4
        w = o.pack_slots([ad], 1, max_rank)[0]
        xa, out = o.lora_delta(w, k_in, n_out, max_rank, _int_bits(x).ravel(), k_in, m,
                               _int_bits(base).ravel(), 0, n_out)
        y = base + 4 * (x @ A.T) @ B.T
        assert np.array_equal(o.bf16_to_f64(out).reshape(m, n_out), y.astype(np.float64))
        assert np.array_equal(o.bf16_to_f64(xa)[:, :rank], (x @ A.T).astype(np.float64))
        assert np.all(xa[:, rank:] == 0)


def pin_lora_delta_matches_routed(o):
    """The pages: the routed fold is byte-identical to row-by-row unrouted calls
    of the same pair.  The matrix form here against the per-row routed oracle with
    every row on one slot, and m rows against m one-row calls, with row strides and
    an output region inside wider rows left untouched outside [0, n_out)."""
    rng = W.rng_for(0, salt=22)
    k_in, n_out, max_rank, m = 72, 40, 16, 11
    ad, w = _one_pair(o, rng, k_in, n_out, 12, max_rank)
    xs, os_, off = k_in + 8, 2 * n_out + 8, n_out
    x = W.bf16_trunc(rng.standard_normal(m * xs).astype(np.float32))
    base = W.bf16_trunc(rng.standard_normal(m * os_).astype(np.float32))
    xa, out = o.lora_delta(w, k_in, n_out, max_rank, x, xs, m, base, off, os_)
    xa_r, out_r = o.bgmv([w], k_in, n_out, max_rank, x, xs, np.zeros(m, np.int32), m, base,
                         off, os_)
    assert np.array_equal(xa, xa_r) and np.array_equal(out, out_r)
    changed = out != base
    inside = np.zeros(m * os_, bool)
    for i in range(m):
        inside[i * os_ + off: i * os_ + off + n_out] = True
        xa1, out1 = o.lora_delta(w, k_in, n_out, max_rank, x[i * xs:], xs, 1,
                                 base[i * os_:(i + 1) * os_], off, os_)
        assert np.array_equal(xa1[0], xa[i])
        assert np.array_equal(out1, out[i * os_:(i + 1) * os_])
    assert np.any(changed) and not np.any(changed & ~inside)
    # m = 0 changes nothing
    xa0, out0 = o.lora_delta(w, k_in, n_out, max_rank, x, xs, 0, base, off, os_)
    assert xa0.shape == (0, max_rank) and np.array_equal(out0, base)


def pin_f16_to_bf16(o):
    """Install-time F16 -> BF16: hand-derived cases, then every F16 pattern
    against torch's float16 -> bfloat16 conversion (NaN: quiet, sign kept)."""
    known = [
        (0x3C00, 0x3F80),  # 1.0
        (0x3C01, 0x3F80),  # 1 + 2^-10: below half a BF16 ulp
        (0x3C04, 0x3F80),  # 1 + 2^-8: tie between 0x3F80 and 0x3F81 -> even
        (0x3C0C, 0x3F82),  # 1 + 3*2^-8: tie between 0x3F81 and 0x3F82 -> even
        (0x3C05, 0x3F81),  # 1 + 2^-8 + 2^-10: just above the tie
        (0x0001, 0x3380),  # smallest subnormal 2^-24, exact in BF16
        (0x03FF, 0x3880),  # largest subnormal (1 - 2^-10) 2^-14 rounds up to 2^-14
        (0x7BFF, 0x4780),  # largest finite 65504 rounds up to 65536
        (0xC000, 0xC000),  # -2
        (0x8000, 0x8000),  # -0
        (0x7C00, 0x7F80),  # +inf
        (0xFC00, 0xFF80),  # -inf
    ]
    for h, b in known:
        assert int(o.f16_to_bf16(np.array([h], np.uint16))[0]) == b, hex(h)
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = o.f16_to_bf16(allh)
    ref = torch.from_numpy(allh.view(np.float16).copy()).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    f = allh.view(np.float16)
    nan = np.isnan(f)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all((mine[nan] & 0x7FC0) == 0x7FC0)
    assert np.array_equal(mine[nan] >> 15, allh[nan] >> 15)


PINS = [pin_bf16_known, pin_bf16_roundtrip, pin_bf16_midpoints, pin_bf16_vs_torch,
        pin_scale_closed_forms, pin_brute_force_bgmv, pin_textbook_lora, pin_pad_invariant,
        pin_inactive_and_strides, pin_batched_equals_rows, pin_fold_order,
        pin_routing_probe_grouped, pin_grouped_invalid_values, pin_routing_probe_gather, pin_window_union, pin_cross_path,
        pin_helpers, pin_lora_delta_brute_force, pin_lora_delta_textbook,
        pin_lora_delta_matches_routed, pin_f16_to_bf16]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)
