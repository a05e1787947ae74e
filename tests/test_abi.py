"""C ABI of librld.so, on the CPU: the library loads, exports every function
include/rld.h declares, its pure host helpers agree with the oracle's
statements of the same helpers, and the device entry points reject bad
arguments with the documented status before any launch.

No device work is done here: every device entry point is called only with
arguments that fail validation, or with an empty batch / empty window (a no-op
that launches nothing), and with stream 0 so no GPU runtime is needed.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle as O
import routed_lora_delta_amd as R

# a fake, 16-byte-aligned "device" address: validation never dereferences it
FAKE = 0x7F0000001000


def test_library_exports_every_header_symbol():
    names = R.header_symbols()
    assert len(names) >= 20, names
    lib = ctypes.CDLL(R.library_path())
    for n in names:
        assert hasattr(lib, n), f"librld.so does not export {n}"
        assert hasattr(R, n), f"the binding has no {n}"
    assert R.rld_version().startswith("rld")
    for st in (R.RLD_OK, R.RLD_EINVAL, R.RLD_EALIGN, R.RLD_EUNSUPPORTED, R.RLD_ELAUNCH,
               R.RLD_ENOSPACE):
        assert R.rld_status_string(st) != "unknown status"


@pytest.mark.parametrize("alpha,rank,rs", [(16.0, 4, 0), (16.0, 8, 0), (32.0, 8, 1),
                                           (32.0, 32, 1), (32.0, 64, 1), (16.0, 3, 0),
                                           (7.0, 48, 1)])
def test_scale_matches_oracle(alpha, rank, rs):
    out = ctypes.c_float()
    assert R.rld_scale(alpha, rank, rs, ctypes.byref(out)) == R.RLD_OK
    assert np.float32(out.value) == O.scale_for(alpha, rank, bool(rs))


def test_scale_rejects_rank_zero():
    out = ctypes.c_float()
    assert R.rld_scale(16.0, 0, 0, ctypes.byref(out)) == R.RLD_EINVAL


@pytest.mark.parametrize("rank,max_rank", [(4, 8), (8, 8), (13, 16), (1, 64)])
def test_pad_adapter_matches_oracle(rank, max_rank):
    rng = np.random.default_rng(rank * 100 + max_rank)
    k_in, n_out = 40, 24
    A = rng.integers(0, 65536, size=(rank, k_in), dtype=np.uint16)
    B = rng.integers(0, 65536, size=(n_out, rank), dtype=np.uint16)
    ap = np.full((max_rank, k_in), 0xFFFF, np.uint16)
    bp = np.full((n_out, max_rank), 0xFFFF, np.uint16)
    assert R.rld_pad_adapter_host(A, B, rank, k_in, n_out, max_rank, ap, bp) == R.RLD_OK
    Ao, Bo = O.pad_adapter(A, B, max_rank)
    assert np.array_equal(ap, Ao) and np.array_equal(bp, Bo)
    assert R.rld_pad_adapter_host(A, B, max_rank + 1, k_in, n_out, max_rank, ap, bp) == \
        R.RLD_EINVAL


def _entries(rows):
    arr = (R.rld_adapter_entry * max(1, len(rows)))()
    for i, (slot, expert, a, b, rank, alpha, rs) in enumerate(rows):
        arr[i] = R.rld_adapter_entry(slot, expert, a, b, rank, alpha, rs)
    return arr


def test_route_pack_last_wins_and_empty_slots():
    rows = [(0, -1, FAKE, FAKE + 256, 8, 16.0, 0),
            (2, -1, FAKE + 512, FAKE + 768, 16, 32.0, 1),
            (0, -1, FAKE + 1024, FAKE + 1280, 4, 16.0, 0)]  # slot 0 again: last wins
    a = np.full(4, 7, np.uint64)
    b = np.full(4, 7, np.uint64)
    s = np.full(4, 7, np.float32)
    assert R.rld_route_pack(_entries(rows), len(rows), 4, 16, a, b, s) == R.RLD_OK
    assert a.tolist() == [FAKE + 1024, 0, FAKE + 512, 0]
    assert b.tolist() == [FAKE + 1280, 0, FAKE + 768, 0]
    assert s[0] == O.scale_for(16.0, 4, False) and s[2] == O.scale_for(32.0, 16, True)
    assert s[1] == 0.0 and s[3] == 0.0


@pytest.mark.parametrize("row,status", [
    ((4, -1, FAKE, FAKE, 8, 16.0, 0), R.RLD_EINVAL),        # slot >= max_loras
    ((1, -1, FAKE, FAKE, 0, 16.0, 0), R.RLD_EINVAL),        # rank 0
    ((1, -1, FAKE, FAKE, 17, 16.0, 0), R.RLD_EINVAL),       # rank > max_rank
    ((1, -1, 0, FAKE, 8, 16.0, 0), R.RLD_EINVAL),           # null address
    ((1, -1, FAKE + 8, FAKE, 8, 16.0, 0), R.RLD_EALIGN),    # misaligned address
])
def test_route_pack_rejects(row, status):
    a = np.zeros(4, np.uint64)
    b = np.zeros(4, np.uint64)
    s = np.zeros(4, np.float32)
    assert R.rld_route_pack(_entries([row]), 1, 4, 16, a, b, s) == status


def test_moe_tables_pack_slot_major():
    E = 5
    rows = [(1, 3, FAKE, FAKE + 256, 8, 16.0, 0), (0, 0, FAKE + 512, FAKE + 768, 16, 16.0, 0),
            (1, 3, FAKE + 1024, FAKE + 1280, 16, 16.0, 0)]
    a = np.zeros(2 * E, np.uint64)
    b = np.zeros(2 * E, np.uint64)
    s = np.zeros(2 * E, np.float32)
    assert R.rld_moe_tables_pack(_entries(rows), 3, 2, E, 16, a, b, s) == R.RLD_OK
    want_a = np.zeros(2 * E, np.uint64)
    want_a[0 * E + 0] = FAKE + 512
    want_a[1 * E + 3] = FAKE + 1024
    assert np.array_equal(a, want_a)
    assert s[1 * E + 3] == O.scale_for(16.0, 16, False)
    bad = [(0, E, FAKE, FAKE, 8, 16.0, 0)]
    assert R.rld_moe_tables_pack(_entries(bad), 1, 2, E, 16, a, b, s) == R.RLD_EINVAL
    bad = [(0, -1, FAKE, FAKE, 8, 16.0, 0)]
    assert R.rld_moe_tables_pack(_entries(bad), 1, 2, E, 16, a, b, s) == R.RLD_EINVAL


@pytest.mark.parametrize("ids", [[3, 0, 7], [5, 5, 1], [0], []])
def test_pack_expert_tables_matches_oracle(ids):
    n = len(ids)
    eids = np.array(ids, np.uint32) if n else np.zeros(1, np.uint32)
    aa = np.array([FAKE + 256 * i for i in range(n)] or [0], np.uint64)
    bb = np.array([FAKE + 4096 + 256 * i for i in range(n)] or [0], np.uint64)
    sc = np.array([0.5 + i for i in range(n)] or [0], np.float32)
    cap = 16
    a = np.zeros(cap, np.uint64)
    b = np.zeros(cap, np.uint64)
    s = np.zeros(cap, np.float32)
    cnt = ctypes.c_uint32(99)
    assert R.rld_pack_expert_tables(eids, aa, bb, sc, n, cap, a, b, s, ctypes.byref(cnt)) == \
        R.RLD_OK
    want = O.pack_expert_tables([(ids[i], aa[i], bb[i], sc[i]) for i in range(n)])
    if want is None:
        assert cnt.value == 0
        return
    ne, wa, wb, ws = want
    assert cnt.value == ne
    assert a[:ne].tolist() == wa and b[:ne].tolist() == wb
    assert np.array_equal(s[:ne], np.array(ws, np.float32))
    cnt2 = ctypes.c_uint32()
    assert R.rld_pack_expert_tables(eids, aa, bb, sc, n, ne - 1, a, b, s,
                                    ctypes.byref(cnt2)) == R.RLD_ENOSPACE


@pytest.mark.parametrize("total,cap", [(0, 8192), (1, 8192), (32768, 8192), (32769, 8192),
                                       (300, 100), (300, 64), (8191, 8192), (5, 1),
                                       # totals and caps near 2^32: no wrap in the ceil
                                       (0xFFFFFFFF, 0x80000000), (0xFFFFFFFF, 0xFFFFFFFF),
                                       (0xFFFFFFFE, 0x7FFFFFFF), (0xFFFFFFFF, 0x10000000)])
def test_grouped_windows_and_wc_match_oracle(total, cap):
    mx = 1024
    st = np.zeros(mx, np.uint32)
    en = np.zeros(mx, np.uint32)
    cnt = ctypes.c_uint32(99)
    assert R.rld_grouped_windows(total, cap, st, en, mx, ctypes.byref(cnt)) == R.RLD_OK
    want = O.grouped_down_windows(total, cap)
    assert cnt.value == len(want)
    assert list(zip(st[:cnt.value].tolist(), en[:cnt.value].tolist())) == want
    for lo, hi in want + [(0, 0), (10, 10)]:
        assert R.rld_grouped_wc(lo, hi) == O.grouped_down_wc(lo, hi)
    if len(want) > 1:
        assert R.rld_grouped_windows(total, cap, st, en, len(want) - 1,
                                     ctypes.byref(cnt)) == R.RLD_ENOSPACE
    assert R.rld_grouped_windows(total, 0, st, en, mx, ctypes.byref(cnt)) == R.RLD_EINVAL


def test_gather_row_token_and_grids():
    for top_k in (1, 4, 8):
        for row in (0, 1, 7, 8, 255, 1000):
            assert R.rld_gather_row_token(row, top_k) == O.gather_row_token(row, top_k)
    g = np.zeros(12, np.uint32)
    assert R.rld_gather_grids(16, 2048, 256, g) == R.RLD_OK
    # one shrink block per flat row; expand covers n_out with whole blocks per row
    assert g[0] == 256 and g[3] * g[4] * g[5] >= 64
    assert g[6] == 256 and g[7] * g[9] * 2 >= 2048


# ------------------------------------------------ device entry points: validation


def _route(k_in=256, n_out=256, max_rank=16, max_loras=4, tables=True):
    t = FAKE if tables else 0
    return R.rld_route(t, t, t, max_loras, k_in, n_out, max_rank)


def _moe_route(k_in=256, n_out=256, max_rank=16, max_loras=2, E=8):
    return R.rld_moe_route(FAKE, FAKE, FAKE, max_loras, E, k_in, n_out, max_rank)


@pytest.mark.parametrize("kw,status", [
    (dict(tables=False), R.RLD_EINVAL),
    (dict(max_loras=0), R.RLD_EINVAL),
    (dict(k_in=0), R.RLD_EINVAL),
    (dict(max_rank=136), R.RLD_EUNSUPPORTED),
    (dict(k_in=250), R.RLD_EALIGN),
    (dict(n_out=100), R.RLD_EALIGN),
    (dict(max_rank=12), R.RLD_EALIGN),
])
def test_bgmv_rejects_bad_routes(kw, status):
    rt = _route(**kw)
    assert R.rld_bgmv_shrink(rt, FAKE, 256, FAKE, 4, FAKE, FAKE, 1 << 20, 0) == status
    assert R.rld_bgmv_expand_fold(rt, FAKE, FAKE, 4, FAKE, 256, 0) == status
    assert R.rld_bgmv(rt, FAKE, 256, FAKE, 4, FAKE, 256, FAKE, FAKE, 1 << 20, 0) == status


def test_bgmv_rejects_bad_buffers():
    rt = _route()
    n = 4
    ws = R.rld_bgmv_workspace_bytes(n, 256, 16, 4)
    sh = lambda **k: R.rld_bgmv_shrink(  # noqa: E731
        rt, k.get("x", FAKE), k.get("xs", 256), k.get("seq", FAKE), n, k.get("xa", FAKE),
        k.get("ws", FAKE), k.get("wsb", ws), 0)
    assert sh(x=0) == R.RLD_EINVAL
    assert sh(xs=128) == R.RLD_EINVAL            # stride < k_in
    assert sh(xs=260) == R.RLD_EALIGN            # stride not a multiple of 8
    assert sh(x=FAKE + 2) == R.RLD_EALIGN        # x not 16-byte aligned
    assert sh(seq=0) == R.RLD_EINVAL
    assert sh(xa=0) == R.RLD_EINVAL
    assert sh(xa=FAKE + 8) == R.RLD_EALIGN
    ex = lambda **k: R.rld_bgmv_expand_fold(  # noqa: E731
        rt, k.get("xa", FAKE), k.get("seq", FAKE), n, k.get("out", FAKE), k.get("os", 256), 0)
    assert ex(out=0) == R.RLD_EINVAL
    assert ex(os=200) == R.RLD_EINVAL            # stride < n_out
    assert ex(out=FAKE + 4) == R.RLD_EALIGN
    assert ex(xa=0) == R.RLD_EINVAL


def test_bgmv_noalloc_rejects_before_touching_the_device():
    """rld_bgmv_noalloc checks its arguments and its scratch limit before any
    HIP call: a call that needs more than RLD_NOALLOC_SCRATCH_BYTES returns
    RLD_ENOSPACE (here, without a GPU, nothing else could run)."""
    assert R.RLD_NOALLOC_SCRATCH_BYTES == 8 << 20
    rt = _route(k_in=12288, n_out=4096, max_rank=64, max_loras=32)

    def call(n, x=FAKE, seq=FAKE, out=FAKE, os_=4096, route=rt):
        return R.rld_bgmv_noalloc(route, x, 12288, seq, n, out, os_, 0)

    def need(n):  # xa arena (256-byte rounded) + the k-split partials
        return -(-n * 64 * 2 // 256) * 256 + R.rld_bgmv_workspace_bytes(n, 12288, 64, 1)

    assert need(1337) <= R.RLD_NOALLOC_SCRATCH_BYTES < need(1338)
    assert call(1338) == R.RLD_ENOSPACE
    assert call(1 << 20) == R.RLD_ENOSPACE
    assert call(0) == R.RLD_OK                      # no-op
    assert call(4, x=0) == R.RLD_EINVAL
    assert call(4, seq=0) == R.RLD_EINVAL
    assert call(4, out=FAKE + 2) == R.RLD_EALIGN
    assert call(4, os_=1000) == R.RLD_EINVAL
    assert call(4, route=_route(tables=False)) == R.RLD_EINVAL


def test_bgmv_multi_rejects_bad_arguments():
    """rld_bgmv_multi checks every route and buffer before any launch."""
    q, k, v = _route(k_in=4096, n_out=4096), _route(k_in=4096, n_out=1024), \
        _route(k_in=4096, n_out=1024)
    n = 64
    wsb = R.rld_bgmv_multi_workspace_bytes(n, 4096, 16, 3)
    assert wsb == 3 * R.rld_bgmv_workspace_bytes(n, 4096, 16, 4)

    def call(routes=(q, k, v), n=n, base=None, os_=None, xa=None, ws=FAKE, wsb=wsb, nr=None,
             x=FAKE, seq=FAKE):
        k_ = len(routes)
        base = [FAKE] * k_ if base is None else base
        os_ = [6144] * k_ if os_ is None else os_
        xa = [FAKE] * k_ if xa is None else xa
        return R.rld_bgmv_multi(list(routes), x, 4096, seq, n, base, os_, xa, ws, wsb,
                                stream=0, nroutes=nr)

    assert call(nr=0) == R.RLD_EINVAL
    assert call(routes=(q, k, v, q, k), nr=5) == R.RLD_EUNSUPPORTED
    assert call(routes=(q, _route(k_in=2048, n_out=1024))) == R.RLD_EINVAL   # k_in differs
    assert call(routes=(q, _route(k_in=4096, max_rank=32))) == R.RLD_EINVAL  # rank differs
    assert call(routes=(q, _route(k_in=4096, tables=False))) == R.RLD_EINVAL
    assert call(n=0) == R.RLD_OK                                   # no-op, nothing launched
    assert call(seq=0) == R.RLD_EINVAL
    assert call(x=FAKE + 2) == R.RLD_EALIGN
    assert call(xa=[FAKE, 0, FAKE]) == R.RLD_EINVAL
    assert call(xa=[FAKE, FAKE + 8, FAKE]) == R.RLD_EALIGN
    assert call(os_=[6144, 1000, 6144]) == R.RLD_EINVAL           # stride < n_out
    assert call(base=[FAKE, FAKE, 0]) == R.RLD_EINVAL
    assert call(wsb=wsb - 16) == R.RLD_ENOSPACE
    assert call(ws=0) == R.RLD_ENOSPACE
    assert call(ws=FAKE + 8) == R.RLD_EALIGN
    # one chunk: no workspace
    assert R.rld_bgmv_multi_workspace_bytes(n, 256, 16, 3) == 0
    assert R.rld_bgmv_multi_workspace_bytes(n, 4096, 16, 0) == 0


def test_bgmv_refuses_launches_past_32_bit_indices():
    """A call whose items or chunk-reduce threads would not fit 32-bit indices
    is refused before any launch (the workspace size passed is large enough)."""
    rt = _route(k_in=4096, n_out=4096, max_rank=128, max_loras=4)
    n = 1 << 26  # 2^26 rows x 32 reduce threads per row
    big = 1 << 62
    assert R.rld_bgmv_shrink(rt, FAKE, 4096, FAKE, n, FAKE, FAKE, big, 0) == R.RLD_EUNSUPPORTED
    assert R.rld_bgmv_multi([rt, rt], FAKE, 4096, FAKE, n, [FAKE] * 2, [4096] * 2, [FAKE] * 2,
                            FAKE, big, stream=0) == R.RLD_EUNSUPPORTED
    pair = R.rld_pair(FAKE, FAKE, 1.0, 4096, 4096, 128)
    assert R.rld_lora_shrink(pair, FAKE, 4096, n, FAKE, FAKE, big, 0) == R.RLD_EUNSUPPORTED


def test_bgmv_workspace_contract():
    # the workspace holds the k-split partials and per-slot bookkeeping; a short
    # one is refused before any launch, by every entry point that takes one
    rt = _route(k_in=12288, n_out=4096, max_rank=64, max_loras=32)
    need = R.rld_bgmv_workspace_bytes(256, 12288, 64, 32)
    # 24 chunks of 512: fp32 partials per row and xa column
    assert need == 24 * 256 * 64 * 4
    for short in (need - 32, need // 2, 16, 0):
        assert R.rld_bgmv_shrink(rt, FAKE, 12288, FAKE, 256, FAKE, FAKE, short, 0) == \
            R.RLD_ENOSPACE
        assert R.rld_bgmv(rt, FAKE, 12288, FAKE, 256, FAKE, 4096, FAKE, FAKE, short, 0) == \
            R.RLD_ENOSPACE
    assert R.rld_bgmv_shrink(rt, FAKE, 12288, FAKE, 256, FAKE, 0, need, 0) == R.RLD_ENOSPACE
    assert R.rld_bgmv_shrink(rt, FAKE, 12288, FAKE, 256, FAKE, FAKE + 8, need, 0) == \
        R.RLD_EALIGN
    # a single chunk needs no workspace at all
    assert R.rld_bgmv_workspace_bytes(4, 256, 64, 2) == 0
    assert R.rld_bgmv_workspace_bytes(256, 0, 64, 32) == 0
    assert R.rld_bgmv_workspace_bytes(256, 4096, 64, 0) == 0


def test_empty_batches_are_noops():
    rt = _route()
    assert R.rld_bgmv(rt, FAKE, 256, FAKE, 0, FAKE, 256, FAKE, FAKE, 0, 0) == R.RLD_OK
    assert R.rld_bgmv_shrink(rt, FAKE, 256, FAKE, 0, FAKE, 0, 0, 0) == R.RLD_OK
    assert R.rld_bgmv_expand_fold(rt, FAKE, FAKE, 0, FAKE, 256, 0) == R.RLD_OK
    mr = _moe_route()
    assert R.rld_moe_gather(mr, FAKE, 256, FAKE, FAKE, 8, 0, FAKE, 256, FAKE, 0) == R.RLD_OK
    # empty grouped window: validated, then nothing to launch
    assert R.rld_moe_grouped(mr, FAKE, 256, 1, 64, FAKE, 8, FAKE, FAKE, 100, 100, FAKE, 256,
                             FAKE, 0, 0, 0, 0) == R.RLD_OK


def test_moe_rejects_bad_arguments():
    mr = _moe_route()
    g = lambda **k: R.rld_moe_grouped_shrink(  # noqa: E731
        k.get("rt", mr), FAKE, 256, k.get("xg", 1), 64, k.get("off", FAKE), k.get("Eo", 8),
        k.get("stid", FAKE), FAKE, k.get("lo", 0), k.get("hi", 64), k.get("xa", FAKE),
        k.get("cap", 64), k.get("ws", 0), k.get("wsb", 0), 0)
    assert g(off=0) == R.RLD_EINVAL
    assert g(Eo=0) == R.RLD_EINVAL
    assert g(lo=10, hi=5) == R.RLD_EINVAL         # row_end < row_offset
    assert g(stid=0) == R.RLD_EINVAL              # x gather needs sorted_token_ids
    assert g(cap=63) == R.RLD_ENOSPACE            # window larger than the xa arena
    assert g(xa=FAKE + 8) == R.RLD_EALIGN
    big = R.rld_moe_route(FAKE, FAKE, FAKE, 64, 128, 256, 256, 16)   # 8192 pairs
    assert g(rt=big) == R.RLD_EUNSUPPORTED
    bad = R.rld_moe_route(FAKE, FAKE, FAKE, 2, 0, 256, 256, 16)
    assert g(rt=bad) == R.RLD_EINVAL
    ga = lambda **k: R.rld_moe_gather_shrink(  # noqa: E731
        mr, k.get("x", FAKE), k.get("xs", 256), FAKE, FAKE, 8, 16, k.get("xa", FAKE), 0)
    assert ga(x=0) == R.RLD_EINVAL
    assert ga(xs=8) == R.RLD_EINVAL
    assert ga(xa=0) == R.RLD_EINVAL
    assert ga(xa=FAKE + 2) == R.RLD_EALIGN


def test_grouped_workspace_contract():
    # k_in = 4096 splits into 8 chunks of 512: fp32 partials per window row, then
    # 16 bytes of counter per (slot, expert) pair; short or missing workspaces
    # are refused before any launch
    need = R.rld_moe_grouped_workspace_bytes(8192, 4096, 32, 4, 128)
    assert need == 8 * 8192 * 32 * 4 + 16 * 4 * 128
    mr = R.rld_moe_route(FAKE, FAKE, FAKE, 4, 128, 4096, 768, 32)
    g = lambda ws, wsb, hi=8192: R.rld_moe_grouped_shrink(  # noqa: E731
        mr, FAKE, 4096, 1, 4096, FAKE, 128, FAKE, FAKE, 0, hi, FAKE, 8192, ws, wsb, 0)
    for short in (need - 16, need // 2, 16):
        assert g(FAKE, short) == R.RLD_ENOSPACE
    assert g(0, need) == R.RLD_EINVAL
    assert g(FAKE + 8, need) == R.RLD_EALIGN
    # a smaller window needs less: the buffer of the largest window serves all
    assert R.rld_moe_grouped_workspace_bytes(100, 4096, 32, 4, 128) == \
        8 * 100 * 32 * 4 + 16 * 4 * 128
    assert g(FAKE, R.rld_moe_grouped_workspace_bytes(100, 4096, 32, 4, 128) - 16, hi=100) == \
        R.RLD_ENOSPACE
    assert R.rld_moe_grouped(mr, FAKE, 4096, 1, 4096, FAKE, 128, FAKE, FAKE, 0, 8192, FAKE, 768,
                             FAKE, 8192, FAKE, need - 16, 0) == R.RLD_ENOSPACE
    # up to k_in = 1024 the whole of k_in is one chunk of four waves, and up to
    # 2048 at max_rank <= 32 one chunk of sixteen waves: no workspace
    assert R.rld_moe_grouped_workspace_bytes(8192, 768, 32, 4, 128) == 0
    assert R.rld_moe_grouped_workspace_bytes(8192, 1024, 32, 4, 128) == 0
    assert R.rld_moe_grouped_workspace_bytes(8192, 2048, 32, 4, 128) == 0
    assert R.rld_moe_grouped_workspace_bytes(64, 1032, 16, 2, 8) == 0
    # past those: chunks of 512
    assert R.rld_moe_grouped_workspace_bytes(64, 1032, 48, 2, 8) == 3 * 64 * 48 * 4 + 16 * 2 * 8
    assert R.rld_moe_grouped_workspace_bytes(64, 2056, 16, 2, 8) == 5 * 64 * 16 * 4 + 16 * 2 * 8
    assert R.rld_moe_grouped_workspace_bytes(64, 4096, 16, 2, 8) == 8 * 64 * 16 * 4 + 16 * 2 * 8
    assert R.rld_moe_grouped_workspace_bytes(8192, 256, 32, 4, 128) == 0
    assert R.rld_moe_grouped_workspace_bytes(8192, 768, 32, 0, 128) == 0


def test_grouped_pair_rejects_bad_arguments():
    # both routes and both outputs are checked before any launch; an empty
    # window is a no-op
    mr = _moe_route()
    pr = lambda **k: R.rld_moe_grouped_pair(  # noqa: E731
        k.get("ra", mr), k.get("rb", mr), FAKE, 256, 1, 64, FAKE, 8, FAKE, FAKE,
        k.get("lo", 0), k.get("hi", 64), k.get("ba", FAKE), k.get("osa", 256), k.get("bb", FAKE),
        k.get("osb", 256), k.get("xa", FAKE), k.get("xb", FAKE), k.get("cap", 64), 0, 0, 0)
    assert pr(lo=100, hi=100) == R.RLD_OK
    assert pr(xb=0) == R.RLD_EINVAL
    assert pr(xa=0) == R.RLD_EINVAL
    assert pr(xb=FAKE + 8) == R.RLD_EALIGN
    assert pr(bb=0) == R.RLD_EINVAL
    assert pr(osb=8) == R.RLD_EINVAL                 # stride below n_out
    assert pr(cap=63) == R.RLD_ENOSPACE
    bad = R.rld_moe_route(FAKE, FAKE, FAKE, 2, 0, 256, 256, 16)
    assert pr(rb=bad) == R.RLD_EINVAL
    big = R.rld_moe_route(FAKE, FAKE, FAKE, 64, 128, 256, 256, 16)   # 8192 pairs
    assert pr(ra=big) == R.RLD_EUNSUPPORTED


def test_lora_rejects_bad_arguments():
    # the unrouted entry points: every argument error is found before a launch
    P = lambda **k: R.rld_pair(k.get("a", FAKE), k.get("b", FAKE), 0.5,  # noqa: E731
                               k.get("k_in", 4096), k.get("n_out", 1024), k.get("r", 16))
    ws = R.rld_lora_workspace_bytes(64, 4096, 16)
    d = lambda p, **k: R.rld_lora_delta(  # noqa: E731
        p, k.get("x", FAKE), k.get("xs", 4096), k.get("m", 64), k.get("out", FAKE),
        k.get("os", 1024), k.get("xa", FAKE), k.get("ws", FAKE), k.get("wsb", ws), 0)
    assert d(P(a=0)) == R.RLD_EINVAL
    assert d(P(b=0)) == R.RLD_EINVAL
    assert d(P(k_in=0)) == R.RLD_EINVAL
    assert d(P(r=136)) == R.RLD_EUNSUPPORTED
    assert d(P(k_in=4092)) == R.RLD_EALIGN
    assert d(P(a=FAKE + 8)) == R.RLD_EALIGN          # A must be 16-byte aligned
    assert d(P(), x=0) == R.RLD_EINVAL
    assert d(P(), xs=1024) == R.RLD_EINVAL            # stride < k_in
    assert d(P(), out=FAKE + 2) == R.RLD_EALIGN
    assert d(P(), os=512) == R.RLD_EINVAL             # stride < n_out
    assert d(P(), xa=0) == R.RLD_EINVAL
    assert d(P(), wsb=ws - 16) == R.RLD_ENOSPACE
    assert d(P(), ws=0) == R.RLD_ENOSPACE
    assert d(P(), m=0) == R.RLD_OK                    # no-op, nothing launched
    assert R.rld_lora_shrink(P(), FAKE, 4096, 0, FAKE, 0, 0, 0) == R.RLD_OK
    assert R.rld_lora_expand_fold(P(), FAKE, 0, FAKE, 1024, 0) == R.RLD_OK
    assert R.rld_lora_expand_fold(P(), 0, 4, FAKE, 1024, 0) == R.RLD_EINVAL
    # the same k split as the routed path, so the same partials
    assert ws == R.rld_bgmv_workspace_bytes(64, 4096, 16, 1) == 16 * 64 * 16 * 4
    assert R.rld_lora_workspace_bytes(64, 256, 16) == 0
    assert R.rld_lora_workspace_bytes(64, 0, 16) == 0


def test_f16_to_bf16_host_matches_oracle_on_every_pattern():
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out = np.zeros_like(allh)
    assert R.rld_f16_to_bf16_host(allh, out, allh.size) == R.RLD_OK
    want = O.f16_to_bf16(allh)
    assert np.array_equal(out, want)
    inplace = allh.copy()                       # src and dst may be the same array
    assert R.rld_f16_to_bf16_host(inplace, inplace, inplace.size) == R.RLD_OK
    assert np.array_equal(inplace, want)
    assert R._lib.rld_f16_to_bf16_host(None, None, 4) == R.RLD_EINVAL
    assert R._lib.rld_f16_to_bf16_host(None, None, 0) == R.RLD_OK


def test_install_peft_f16_pair_matches_oracle():
    # PEFT F16 tensors -> BF16 -> pool layout, and the scale, against the
    # oracle's conversion, padding and scale
    from routed_lora_delta_amd.pool import install_peft_pair
    rng = np.random.default_rng(5)
    rank, k_in, n_out, max_rank = 12, 40, 24, 16
    a16 = (rng.standard_normal((rank, k_in)) * 0.1).astype(np.float16).view(np.uint16)
    b16 = (rng.standard_normal((n_out, rank)) * 0.02).astype(np.float16).view(np.uint16)
    a_pad, b_pad, sc = install_peft_pair(a16, b16, rank, k_in, n_out, max_rank, 32.0, True)
    wa, wb = O.pad_adapter(O.f16_to_bf16(a16), O.f16_to_bf16(b16), max_rank)
    assert np.array_equal(a_pad, wa) and np.array_equal(b_pad, wb)
    assert sc == O.scale_for(32.0, rank, True)


def test_scale_table_values_are_exact_closed_forms():
    # the fp32 scales of the decode workloads: alpha/r and alpha/sqrt(r), rounded once
    for alpha, r in ((32.0, 8), (32.0, 32), (16.0, 16)):
        out = ctypes.c_float()
        R.rld_scale(alpha, r, 1, ctypes.byref(out))
        assert out.value == float(np.float32(alpha / math.sqrt(r)))


def test_bgmv_launch_count():
    """rld_bgmv's launch count: one in the one-pass form (max_rank <= 16,
    k_in <= 4096, n <= 256, at most 256 (slot, 512-column) items over the
    routes), three with a k_in split, two without one, zero for an empty
    batch or routes the calls reject."""
    L = R.rld_bgmv_launches
    q = _route(4096, 4096, 16, 16)                     # 8 x 16 = 128 items
    kv = _route(4096, 1024, 16, 16)                    # 2 x 16 = 32
    assert L(q, 64) == 1 and L(q, 256) == 1 and L(q, 257) == 3
    assert L([q, kv, kv], 64) == 1                     # 192 items
    assert L([q, q, kv], 64) == 3                      # 288 items
    assert L(_route(4096, 12288, 16, 16), 64) == 3     # 384 items
    assert L(_route(8192, 4096, 16, 16), 64) == 3      # k_in above 16 chunks
    assert L(_route(4096, 12288, 64, 32), 256) == 3    # rank 64
    assert L(_route(200, 264, 8, 3), 5) == 1           # one chunk shorter than 256
    assert L(_route(512, 768, 64, 4), 64) == 2         # rank 64, one 512 chunk
    assert L(_route(256, 264, 16, 4), 300) == 2
    assert L(q, 0) == 0
    assert L(_route(4096, 4096, 16, 16, tables=False), 64) == 0
    assert L([q, _route(4096, 4096, 24, 16)], 64) == 0  # different max_rank
