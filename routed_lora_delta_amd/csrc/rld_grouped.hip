// MoE grouped fold over one chunk window [row_offset, row_end) of expert-sorted
// rows ("Module moe_lora_grouped", moe_lora_grouped_down).
//
// Row r of the window belongs to the expert e whose span of the expert_offsets
// prefix sum holds it (off[e] <= r < off[e+1]); its adapter slot is
// row_adapter[sorted_token_ids[r]] (slot 0 without row_adapter).  The fold of a
// row uses the pair (slot, expert): xa = bf16(x_row @ A_{s,e}^T), then
// base_out[r] += scale * bf16(xa @ B_{s,e}^T).
//
// Work is keyed on the pair, not on fixed row tiles: the work item of pair
// (s, e) reads the window part of expert e's span, keeps the rows whose slot is
// s, and streams a k chunk of A_{s,e} (shrink) or a column slice of B_{s,e}
// (expand) exactly once for all of them.  Every piece of an x row or a base
// row is touched by one item, and the MFMA jobs are as tall as the pair's row
// count.
// Launches are persistent: a fixed number of blocks (host constant, so a
// captured launch keeps its shape), each of which lists the window's active
// pairs (adapter present, rows in the window) from the offsets and the tables
// in one round of loads, then takes its share of the items.  No block is spent
// on a pair that has nothing to do.
//
// The shrink spreads each pair over the whole chip: its items are (pair, k
// chunk), so the pair's A_{s,e} and x rows are streamed by several blocks at
// once, and fp32 partial sums per chunk meet in a workspace (see GsArgs).
//
// Summation order.  The shrink cuts k_in into chunks of a length fixed by
// (k_in, max_rank) alone, each chunk into four (sixteen in the wide case) wave
// ranges; a wave sums its range in one MFMA chain, the wave sums are added in
// wave order and the chunk sums in chunk order.  The expand is one MFMA chain over max_rank.  A row's result
// therefore never depends on which other rows share its block or window: a
// full-window call and the union of chunk windows are bit-identical.
//
// xa rows of window rows that do not fold are written as zeros by row-block
// items of the shrink.
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

// LDS worklist capacities of a launch: PC pairs (max_loras * num_experts) and
// off_cap<PC>() staged expert_offsets entries (num_experts_off < off_cap).  A
// launch uses the small instantiation whenever the route fits it: its prologue
// issues a quarter of the loads and its block holds less LDS, which shortens
// both the first round trip and the launch ramp.
constexpr int kPairCapSmall = 512;
constexpr int kPairCapLarge = 2048;
template <int PC>
constexpr int off_cap() { return PC < 1024 ? PC : 1024; }
constexpr int kListCap = 512;    // rows of a pair collected per scan
constexpr int kBatch = 64;       // rows of a pair per MFMA pass (4 subtiles of 16)
constexpr int kPeThreads = 512;  // expand block: 8 waves x 64 columns
constexpr int kPeCols = 512;     // output columns per expand item
constexpr int kPeGrid = 512;     // expand blocks per launch
constexpr int kDlStride = kPeCols + 8;

// Routing inputs of a window; device addresses are integers read through the
// global-pointer accessors (see gp()).
struct GroupedRows {
  uint64_t off_, stid_, radapt_, atab_, btab_;
  uint32_t E_off;
  uint32_t num_tokens;
  uint32_t max_loras;
  uint32_t E;
  int need_tok;
  __device__ const RLD_GLOBAL int32_t* off() const { return gp<const int32_t>(off_); }
  __device__ const RLD_GLOBAL int32_t* stid() const { return gp<const int32_t>(stid_); }
  __device__ const RLD_GLOBAL int32_t* radapt() const { return gp<const int32_t>(radapt_); }
  __device__ const RLD_GLOBAL uint64_t* a_table() const { return gp<const uint64_t>(atab_); }
  __device__ const RLD_GLOBAL uint64_t* b_table() const { return gp<const uint64_t>(btab_); }
};

// Window part [lo, hi) of expert e's span (empty when e has no offsets entry).
__device__ __forceinline__ void span_in_window(const int* off, const GroupedRows& g, int e,
                                               uint32_t row_offset, uint32_t row_end,
                                               uint32_t& lo, uint32_t& hi) {
  lo = hi = row_end;
  if ((uint32_t)e >= g.E_off) return;
  const int a = off[e], b = off[e + 1];
  // integer clamps to the window (a negative bound counts as 0, so a span
  // ending below zero is empty)
  lo = (a < 0 || (uint32_t)a < row_offset) ? row_offset : (uint32_t)a;
  hi = b < 0 ? 0u : ((uint32_t)b < row_end ? (uint32_t)b : row_end);
  if (hi < lo) hi = lo;
}

// Adapter slot of token t (in range): slot 0 without row_adapter, else its
// row_adapter entry.
__device__ __forceinline__ int token_slot(const GroupedRows& g, int t) {
  return g.radapt_ ? g.radapt()[t] : 0;
}

// Adapter slot of sorted row r, or -1 when its token is out of range; the
// token goes to *tok.
__device__ __forceinline__ int row_slot(const GroupedRows& g, uint32_t r, int* tok) {
  int t = 0;
  if (g.need_tok) {
    t = g.stid()[r];
    if (t < 0 || (uint32_t)t >= g.num_tokens) return -1;
  }
  *tok = t;
  return token_slot(g, t);
}

// Appends to list/toks (LDS) the rows of [c0, c1) (c1 - c0 <= blockDim) that
// expert e owns and whose slot is s, in ascending order; returns how many.
// Called by every thread.
__device__ __forceinline__ int append_pair_rows(const GroupedRows& g, const int* off, int e,
                                                int s, uint32_t c0, uint32_t c1, int* list,
                                                int* toks, int base, int* wcount) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t r = c0 + threadIdx.x;
  bool hit = false;
  int t = 0;
  if (r < c1 && expert_of_row(off, (int)g.E_off, (int)r) == e) hit = row_slot(g, r, &t) == s;
  const uint64_t m = __ballot(hit);
  if (lane == 0) wcount[wave] = __popcll(m);
  __syncthreads();
  int pos = base;
  int tot = 0;
  for (int v = 0; v < nw; ++v) {
    pos += v < wave ? wcount[v] : 0;
    tot += wcount[v];
  }
  if (hit) {
    const int p = pos + __popcll(m & lanemask_lt(lane));
    list[p] = (int)r;
    toks[p] = t;
  }
  __syncthreads();
  return tot;
}

__device__ __forceinline__ void zero_xa_row(RLD_GLOBAL uint16_t* xa, uint32_t local_row,
                                            uint32_t R) {
  // R is a nonzero multiple of 8 (the host checks it): no guard before the first store
  uint32_t i = 0;
#pragma unroll 1
  do {
    store16(xa + (size_t)local_row * R + 8 * i, zero16());
  } while (++i < R / 8);
}

// Every thread (NTH of them): stage expert_offsets in LDS, read the A/B table entries of every pair
// (valid[p] = both present), and list in LDS, ascending, the pairs that are
// valid and own rows of [row_offset, row_end).  With KEEP & 1 it also keeps
// every pair's A table entry in k0.a, with KEEP & 2 its B entry in k0.b and its
// scale (k0.scale_table) in k0.scale, so that an item has its operand addresses
// without a round trip of its own.  NR = 2 (a launch folding two routes that
// share the routing) reads the second route's tables k1.at, k1.bt and
// k1.scale_table too and keeps them in k1.a, k1.b, k1.scale; valid[p] then has
// bit r set when route r adapts pair p, and a pair is listed when either does.
// All these loads go out together, so this costs one round of loads.  Returns
// the pair count.
struct PairKeep {
  uint64_t* a = nullptr;
  uint64_t* b = nullptr;
  float* scale = nullptr;
  const RLD_GLOBAL float* scale_table = nullptr;
  const RLD_GLOBAL uint64_t* at = nullptr;  // second route's tables (NR = 2)
  const RLD_GLOBAL uint64_t* bt = nullptr;
};

template <int NTH, int PC, int KEEP = 0, int NR = 1>
__device__ __forceinline__ int build_worklist(const GroupedRows& g, uint32_t row_offset,
                                              uint32_t row_end, int* off_s, uint8_t* valid,
                                              int16_t* apairs, int* wcount,
                                              const PairKeep& k0 = PairKeep{},
                                              const PairKeep& k1 = PairKeep{}) {
  constexpr int kOffPer = (off_cap<PC>() + NTH - 1) / NTH;
  constexpr int kPairPer = (PC + NTH - 1) / NTH;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int nw = NTH / kWave;
  const uint32_t np = g.max_loras * g.E;
  int ov[kOffPer];
  uint64_t ta[kPairPer], tb[kPairPer];
  float sv[kPairPer];
  uint64_t ta2[NR == 2 ? kPairPer : 1], tb2[NR == 2 ? kPairPer : 1];
  float sv2[NR == 2 ? kPairPer : 1];
#pragma unroll
  for (int i = 0; i < kOffPer; ++i) {
    const uint32_t j = threadIdx.x + i * NTH;
    ov[i] = g.off()[j <= g.E_off ? j : 0];
  }
  // unconditional loads at clamped indices: a load under a branch gets a wait
  // of its own, which would serialise this round
#pragma unroll
  for (int i = 0; i < kPairPer; ++i) {
    const uint32_t p = threadIdx.x + i * NTH;
    const uint32_t pc = p < np ? p : 0;
    ta[i] = g.a_table()[pc];
    tb[i] = g.b_table()[pc];
    if (KEEP & 2) sv[i] = k0.scale_table[pc];
    if (NR == 2) {
      ta2[i] = k1.at[pc];
      tb2[i] = k1.bt[pc];
      sv2[i] = k1.scale_table[pc];
    }
  }
#pragma unroll
  for (int i = 0; i < kOffPer; ++i) {
    const uint32_t j = threadIdx.x + i * NTH;
    if (j <= g.E_off) off_s[j] = ov[i];
  }
#pragma unroll
  for (int i = 0; i < kPairPer; ++i) {
    const uint32_t p = threadIdx.x + i * NTH;
    if (p < np) {
      uint8_t v = (ta[i] != 0ull && tb[i] != 0ull) ? 1 : 0;
      if (NR == 2) v |= (ta2[i] != 0ull && tb2[i] != 0ull) ? 2 : 0;
      valid[p] = v;
      if (KEEP & 1) k0.a[p] = ta[i];
      if (KEEP & 2) {
        k0.b[p] = tb[i];
        k0.scale[p] = sv[i];
      }
      if (NR == 2) {
        k1.a[p] = ta2[i];
        k1.b[p] = tb2[i];
        k1.scale[p] = sv2[i];
      }
    }
  }
  __syncthreads();
  const int* off = off_s;
  int na = 0;
  for (uint32_t c0 = 0; c0 < np; c0 += NTH) {
    const uint32_t p = c0 + threadIdx.x;
    bool act = false;
    if (p < np && valid[p]) {
      uint32_t lo, hi;
      span_in_window(off, g, (int)(p % g.E), row_offset, row_end, lo, hi);
      act = hi > lo;
    }
    const uint64_t m = __ballot(act);
    if (lane == 0) wcount[wave] = __popcll(m);
    __syncthreads();
    int pos = na;
    int tot = 0;
#pragma unroll
    for (int v = 0; v < nw; ++v) {
      pos += v < wave ? wcount[v] : 0;
      tot += wcount[v];
    }
    if (act) apairs[pos + __popcll(m & lanemask_lt(lane))] = (int16_t)p;
    na += tot;
    __syncthreads();
  }
  return na;
}

// Shrink work items of the chunked kernel (256-thread blocks), in this order:
//   (active pair p, k chunk c, column group cg)  for p < na, c < nch, cg < ncg
//   row block z of the window (256 rows)         for z < nz
// A pair item streams chunk c of x and of A_{s,e} for the pair's rows: wave w
// of the block sums k range [c*kc + w*kc/4, c*kc + (w+1)*kc/4) (KS MFMA steps
// of 32) for up to 64 rows at a time, and the four wave sums meet in LDS in
// wave order.  With one chunk that sum is rounded to xa right away; otherwise
// it goes to the fp32 partials part[c][local row][column], and the block that
// completes the pair's last item (a per-pair counter at the end of the
// workspace) adds the chunks in chunk order and writes xa.  An item covers
// NT*16 xa columns (column group cg).  A row-block item zeroes the xa rows of
// its 256 rows that no pair folds.  The wide kernel's items are listed with it
// below.
struct GsArgs {
  uint64_t x_, xa_, part_, ctr_;
  uint64_t out_, scale_;  // fused kernel: base_out and the scale table
  uint32_t n_out, os;     // fused kernel: output width and row stride
  // pair kernel: the second projection's xa, output, tables
  uint64_t xa2_, out2_, scale2_, atab2_, btab2_;
  uint32_t n_out2, os2;
  GroupedRows gr;
  uint32_t xs, x_gather, k_in, R, row_offset, row_end;
  uint32_t kc;   // k chunk: 4 waves x 32*KS (16 waves x 128 in the wide kernel)
  uint32_t nch;  // chunks, ceil(k_in / kc)
  uint32_t ncg;  // column groups, ceil(R / (16*NT))
  uint32_t nz;   // row blocks of the window (of blockDim rows)
  __device__ const RLD_GLOBAL uint16_t* x() const { return gp<const uint16_t>(x_); }
  __device__ RLD_GLOBAL uint16_t* xa() const { return gp<uint16_t>(xa_); }
  __device__ RLD_GLOBAL float* part() const { return gp<float>(part_); }
  __device__ RLD_GLOBAL uint16_t* out() const { return gp<uint16_t>(out_); }
  __device__ const RLD_GLOBAL float* scale_table() const { return gp<const float>(scale_); }
  // 16 bytes per pair, below the end of the workspace
  __device__ RLD_GLOBAL uint32_t* ctr(int pair) const {
    return gp<uint32_t>(ctr_) - 4 * (pair + 1);
  }
};

constexpr int kGsThreads = 256;   // block of the chunked kernel
constexpr int kGsWaves = kGsThreads / kWave;
constexpr int kGwThreads = 1024;  // block of the wide kernel
constexpr int kGwWaves = kGwThreads / kWave;

// LDS of a shrink block of NTH threads.  A gs_scan round takes RPT rows per
// thread (at least 512 rows a round, so that an expert's span of the window,
// about te / num_experts rows, is usually one round), and the row list holds
// one round.
template <int PC, int NTH>
struct GsSmem {
  static constexpr int kNW = NTH / kWave;
  static constexpr int kRPT = NTH >= 512 ? 1 : 512 / NTH;
  static constexpr int kRound = NTH * kRPT;
  uint64_t atab[PC];  // A table entry of every pair
  int off[off_cap<PC>()];
  uint8_t valid[PC];
  int16_t apairs[PC];
  int list[kRound];  // sorted rows of the pair
  int xrow[kRound];  // their x rows (token, or the sorted row)
  int wcount[kRPT * kNW];
  int flag;
};

// One round of gs_scan: the rows of [c0, min(c0 + SM::kRound, hi)) that
// expert e owns and whose adapter slot is s are appended at sm.list[cnt..] in
// row order.  A thread takes rows c0 + tid, c0 + NTH + tid, ...; the loads of
// all of them go out together (clamped, in-bounds indices), so a round is two
// dependent loads whatever its length.  Returns the rows appended.
template <class SM>
__device__ __forceinline__ int gs_round(const GroupedRows& g, SM& sm, int e, int s, uint32_t c0,
                                        uint32_t hi, uint32_t x_gather, int cnt) {
  constexpr int RPT = SM::kRPT, NW = SM::kNW, NTH = NW * kWave;
  // The thread index passes through an empty asm, so that the lane masks and
  // LDS addresses below are computed at each round rather than hoisted out of
  // the callers' item loops, where they would hold registers throughout.
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t r[RPT];
  bool hit[RPT];
  int t[RPT], sr[RPT];
#pragma unroll
  for (int h = 0; h < RPT; ++h) {
    r[h] = c0 + (uint32_t)(h * NTH) + (uint32_t)tid;
    hit[h] = r[h] < hi && expert_of_row(sm.off, (int)g.E_off, (int)r[h]) == e;
    t[h] = (int)r[h];
    sr[h] = 0;
  }
  if (g.need_tok) {
#pragma unroll
    for (int h = 0; h < RPT; ++h) t[h] = g.stid()[r[h] < hi ? r[h] : c0];
#pragma unroll
    for (int h = 0; h < RPT; ++h) hit[h] = hit[h] && t[h] >= 0 && (uint32_t)t[h] < g.num_tokens;
  }
  if (g.radapt_ && g.num_tokens > 0) {
#pragma unroll
    for (int h = 0; h < RPT; ++h) sr[h] = g.radapt()[hit[h] ? t[h] : 0];
  }
  uint64_t m[RPT];
#pragma unroll
  for (int h = 0; h < RPT; ++h) {
    hit[h] = hit[h] && sr[h] == s;
    m[h] = __ballot(hit[h]);
    if (lane == 0) sm.wcount[h * NW + wave] = __popcll(m[h]);
  }
  __syncthreads();
  int pos[RPT];
  int acc = cnt;
#pragma unroll
  for (int h = 0; h < RPT; ++h) {
    int before = 0, all = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int wc = sm.wcount[h * NW + v];
      before += v < wave ? wc : 0;
      all += wc;
    }
    pos[h] = acc + before;
    acc += all;
  }
#pragma unroll
  for (int h = 0; h < RPT; ++h)
    if (hit[h]) {
      const int p = pos[h] + __popcll(m[h] & lanemask_lt(lane));
      sm.list[p] = (int)r[h];
      sm.xrow[p] = x_gather ? t[h] : (int)r[h];
    }
  __syncthreads();
  return acc - cnt;
}

// Collects into sm.list / sm.xrow the rows of [*c0, hi) that expert e owns and
// whose adapter slot is s, up to one round's worth (rounds that find nothing
// do not end the segment), and advances *c0 past the rows scanned (*c0 < hi on
// entry).  Every thread calls it; returns the row count.
template <class SM>
__device__ __forceinline__ int gs_scan(const GroupedRows& g, SM& sm, int e, int s, uint32_t* c0,
                                       uint32_t hi, uint32_t x_gather) {
  int cnt = 0;
  do {
    cnt += gs_round(g, sm, e, s, *c0, hi, x_gather, cnt);
    *c0 += SM::kRound;
  } while (*c0 < hi && cnt == 0);
  return cnt;
}

// Last block of a pair: xa[row, :] = bf16(sum over chunks, in chunk order, of
// the partials) for the cnt rows in sm.list.  Each thread takes up to 4 column
// pairs; all their chunk loads (up to 8 chunks at a time) go out before the
// adds.
template <int PC>
__device__ __forceinline__ void gs_reduce_rows(const GsArgs& a, const GsSmem<PC, kGsThreads>& sm,
                                               int cnt) {
  const uint32_t R = a.R;
  const uint32_t half = R / 2;
  const size_t W = a.row_end - a.row_offset;
  const size_t cstride = W * R / 2;  // uint64 per chunk
  const uint32_t tot = (uint32_t)cnt * half;
  const RLD_GLOBAL uint64_t* part = reinterpret_cast<const RLD_GLOBAL uint64_t*>(a.part());
  for (uint32_t base = 0; base < tot; base += 4 * kGsThreads) {
    uint32_t off[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t ei = base + threadIdx.x + u * kGsThreads;
      ok[u] = ei < tot;
      const uint32_t li = ok[u] ? ei / half : 0;
      const uint32_t lr = (uint32_t)sm.list[li] - a.row_offset;
      off[u] = lr * half + (ok[u] ? ei % half : 0);
    }
    float s0[4], s1[4];
    for (uint32_t cb = 0; cb < a.nch; cb += 8) {
      uint64_t v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[u][j] = (ok[u] && cb + j < a.nch)
                        ? __hip_atomic_load(part + (cb + j) * cstride + off[u], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : 0ull;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f0 = __uint_as_float((uint32_t)v[u][j]);
          const float f1 = __uint_as_float((uint32_t)(v[u][j] >> 32));
          if (cb + j == 0) {
            s0[u] = f0;
            s1[u] = f1;
          } else if (cb + j < a.nch) {
            s0[u] += f0;
            s1[u] += f1;
          }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ok[u])
        *reinterpret_cast<RLD_GLOBAL uint32_t*>(a.xa() + 2 * (size_t)off[u]) =
            pack_bf16x2(s0[u], s1[u]);
  }
}

// Pair item (pair, chunk c, column group cg); see GsArgs.  h = 0 or 1 (one
// chunk and one column group only): the item takes the first ceil(cnt / 2) or
// the remaining rows of each scan round; h < 0: all of them.
template <int KS, int NT, int PC>
__device__ void gs_pair_item(const GsArgs& a, GsSmem<PC, kGsThreads>& sm, floatx4 (*red)[4 * NT][kWave], int pair,
                             uint32_t c, uint32_t cg, int h = -1) {
  const GroupedRows& g = a.gr;
  const uint32_t R = a.R, k_in = a.k_in;
  const int s = pair / (int)g.E;
  const int e = pair % (int)g.E;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t kw0 = c * a.kc + (uint32_t)wave * (32u * KS);
  const uint32_t col0 = cg * 16u * NT;
  uint32_t lo, hi;
  span_in_window(sm.off, g, e, a.row_offset, a.row_end, lo, hi);

  const uint64_t ta = sm.atab[pair];
  uint32_t c0 = lo;
  int cnt = gs_scan(g, sm, e, s, &c0, hi, a.x_gather);
  // Every item of the pair finds the same rows; a pair without rows (no row
  // of e's span is on slot s) has nothing to write or count.
  if (cnt == 0) return;
  const bool multi = c0 < hi;

  const RLD_GLOBAL uint16_t* x = a.x();
  const bool one_chunk = a.nch == 1;
  const size_t W = a.row_end - a.row_offset;
  // up to 64 rows of the segment, starting at b0, below bend
  const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(ta);
  int bend = cnt;
  auto batch = [&](int b0) {
    const int nb = min(bend - b0, 64);
    // Rows col0.. of A_{s,e} over this wave's k range (MFMA B operands) and the
    // x rows of the batch's four 16-row subtiles, all in one round of loads
    // (clamped in-bounds addresses).
    uint4 bop[NT][KS];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t col = col0 + 16u * j + cl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kk = kw0 + 32u * ks + 8u * lg;
        bop[j][ks] = load16(A + (col < R && kk < k_in ? (size_t)col * k_in + kk : 0));
      }
    }
    uint4 aop[4][KS];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int li = q * 16 + cl;
      const RLD_GLOBAL uint16_t* xr = x + (size_t)sm.xrow[b0 + (li < nb ? li : 0)] * a.xs;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kk = kw0 + 32u * ks + 8u * lg;
        aop[q][ks] = load16(xr + (kk < k_in ? kk : 0));
      }
    }
    issue_point();
    // k past k_in contributes nothing (both operands zeroed); columns past
    // max_rank are computed from clamped reads and never stored
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      if (kw0 + 32u * ks + 8u * lg >= k_in) {
#pragma unroll
        for (int q = 0; q < 4; ++q) aop[q][ks] = zero16();
#pragma unroll
        for (int j = 0; j < NT; ++j) bop[j][ks] = zero16();
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16_16x16x32(aop[q][ks], bop[j][ks], acc);
        red[wave][q * NT + j][lane] = acc;
      }
    __syncthreads();
    {
      // one thread per (subtile, lane): the wave sums in wave order
      const int q = threadIdx.x >> 6;
      const int ln = threadIdx.x & 63;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint32_t col = col0 + 16u * j + (ln & 15);
        floatx4 sum = red[0][q * NT + j][ln];
#pragma unroll
        for (int v = 1; v < kGsWaves; ++v) sum += red[v][q * NT + j][ln];
        if (col < R) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int li = q * 16 + 4 * (ln >> 4) + i;
            if (li < nb) {
              const uint32_t lr = (uint32_t)sm.list[b0 + li] - a.row_offset;
              if (one_chunk)
                a.xa()[(size_t)lr * R + col] = (uint16_t)f32_to_bf16(sum[i]);
              else
                __hip_atomic_store(a.part() + ((size_t)c * W + lr) * R + col, sum[i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    __syncthreads();
  };
  // Each scan round's rows [b1, bend): all of them, or this item's half.
  for (;;) {
    const int split = (cnt + 1) / 2;
    const int b1 = h > 0 ? split : 0;
    bend = h == 0 ? split : cnt;
    if (bend - b1 <= 64) {
      if (b1 < bend) batch(b1);  // the usual case
    } else {
      for (int b0 = b1; b0 < bend; b0 += 64) batch(b0);
    }
    if (c0 >= hi) break;
    cnt = gs_scan(g, sm, e, s, &c0, hi, a.x_gather);
  }
  if (one_chunk) return;

  // The block that completes the pair adds the chunks.
  RLD_GLOBAL uint32_t* ctr = a.ctr(pair);
  if (block_signal(ctr, &sm.flag) != a.nch * a.ncg - 1) return;
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!multi) {  // sm.list still holds the pair's rows
    gs_reduce_rows(a, sm, cnt);
    return;
  }
  c0 = lo;
  while (c0 < hi) {
    cnt = gs_scan(g, sm, e, s, &c0, hi, a.x_gather);
    gs_reduce_rows(a, sm, cnt);
  }
}

// Row-block item z of a block of NTH threads: zero the xa rows of
// [row_offset + NTH z, +NTH) that no pair folds (no owner expert, token out of
// range, slot out of range or not adapted for the expert).
template <int PC, int NTH>
__device__ __forceinline__ void gs_zero_item(const GsArgs& a, const GsSmem<PC, NTH>& sm,
                                             uint32_t z, uint64_t xa2 = 0) {
  const GroupedRows& g = a.gr;
  // the thread index passes through an empty asm, so that the row addresses
  // below are computed here and not hoisted into the callers' item loops
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const uint32_t r = a.row_offset + z * NTH + (uint32_t)tid;
  if (r >= a.row_end) return;
  const int e = expert_of_row(sm.off, (int)g.E_off, (int)r);
  bool fold = e >= 0 && (uint32_t)e < g.E;
  int t = 0;
  if (fold && g.need_tok) {
    t = g.stid()[r];
    fold = t >= 0 && (uint32_t)t < g.num_tokens;
  }
  int s = 0;
  if (fold) s = token_slot(g, t);
  fold = fold && s >= 0 && (uint32_t)s < g.max_loras && sm.valid[s * (int)g.E + e];
  if (!fold) {
    zero_xa_row(a.xa(), r - a.row_offset, a.R);
    if (xa2) zero_xa_row(gp<uint16_t>(xa2), r - a.row_offset, a.R);
  }
}

// Persistent: every block lists the window's active pairs, then takes items
// blockIdx.x, blockIdx.x + gridDim.x, ...
template <int KS, int NT, int PC>
__global__ __launch_bounds__(kGsThreads) void grouped_shrink_kernel(GsArgs a) {
  __shared__ GsSmem<PC, kGsThreads> sm;
  __shared__ floatx4 red[kGsWaves][4 * NT][kWave];
  PairKeep k0;
  k0.a = sm.atab;
  const int na = build_worklist<kGsThreads, PC, 1>(a.gr, a.row_offset, a.row_end, sm.off,
                                                   sm.valid, sm.apairs, sm.wcount, k0);
  // One chunk and one column group: items (pair, row half), both halves of a
  // pair on one XCD (item it runs on a block with blockIdx.x = it mod
  // gridDim.x, a multiple of 8), whose L2 serves the second read of A_{s,e}.
  // Otherwise (pair, chunk, column group).  Then the row blocks.
  const bool halves = a.nch == 1 && a.ncg == 1;
  const uint32_t per = a.nch * a.ncg;
  const uint32_t npi = halves ? 16u * (((uint32_t)na + 7u) / 8u) : (uint32_t)na * per;
  const uint32_t total = npi + a.nz;
  for (uint32_t it = blockIdx.x; it < total; it += gridDim.x) {
    if (it < npi) {
      uint32_t p = it / per, c = 0, cg = 0;
      int h = -1;
      if (halves) {
        p = (it / 16u) * 8u + it % 8u;
        h = (int)((it / 8u) % 2u);
      } else {
        c = (it % per) / a.ncg;
        cg = (it % per) % a.ncg;
      }
      if (p < (uint32_t)na) gs_pair_item<KS, NT, PC>(a, sm, red, sm.apairs[p], c, cg, h);
    } else {
      gs_zero_item(a, sm, it - npi);
    }
  }
}

// Wide kernel (1024 < k_in <= 2048, max_rank <= 32): blocks of 16 waves, one
// chunk.  Items, in this order:
//   (active pair p, row half h)  for p < na, h < 2, ordered so that both halves
//                                of a pair have the same blockIdx % 8 (so the
//                                same XCD, whose L2 then serves the second read
//                                of A_{s,e})
//   row block z of the window (1024 rows)
// Of the c rows the scan finds for the pair, item (p, 0) takes the first
// ceil(c / 2) and item (p, 1) the rest, in batches of up to 16 kWideQB rows (a
// pair of up to 96 rows is one batch per half): wave w sums k range
// [128w, 128w + 128) in one MFMA chain of four steps for all NT*16 xa columns,
// the 16 wave sums meet in LDS in wave order, and the sum is rounded to xa.
// A batch's first 32 x rows and A_{s,e} over the wave's range are one round of
// loads (A_{s,e} whole, 128 KB at max_rank 32, and 32 x 4 KB of x rows in
// flight per block); rows 32..47 are a second round.
//
// FUSE (grouped_fold_wide_kernel, n_out <= kFuseCols): the block then folds the
// batch's rows right away, the expand of the same pair on the xa it has just
// rounded: each wave's kFuseTiles 16-column tiles of B_{s,e} (MFMA A operands,
// one k step of 32 covers max_rank), the batch's base rows and the xa tile
// (from LDS) in one round, deltas -> LDS (over the wave-sum buffer) -> 16-byte
// fold of the base rows.  The expand's own launch, row scan and xa round trip
// through memory are saved.
constexpr int kWideQB = 3;  // 16-row subtiles per batch of the wide kernels
constexpr int kFuseTiles = 3;
constexpr int kFuseCols = kGwWaves * kFuseTiles * 16;  // 768
constexpr int kFuseStride = kFuseCols + 8;             // LDS row stride of the delta tile
constexpr int kXlStride = 32 + 8;                       // LDS row stride of the xa tile

// Fused fold of a batch of up to 16*FQ rows (see gs_wide_item): rows[0, nb)
// of the sorted rows, their xa (BF16, max_rank <= 32 columns) in xl, deltas
// staged in dl, n_out <= kFuseCols.  Every thread of the 1024 calls it.  The
// fold's global operands (each wave's B tiles, the base pieces) go out in
// wide_fold_issue, which may run ahead of the wave sums that write xl;
// wide_fold_finish reads xl and folds.
// 16-byte base pieces per thread for a fold of FQ 16-row subtiles
template <int FQ>
constexpr int fold_pieces() { return (16 * FQ * (kFuseCols / 8) + kGwThreads - 1) / kGwThreads; }
struct FoldOps {
  uint4 bt[kFuseTiles];
  uint4 bv[fold_pieces<3>()];
};

template <bool ISSUE_B = true, bool ISSUE_BASE = true, int FQ = 2>
__device__ __forceinline__ void wide_fold_issue(uint64_t out_addr, uint32_t os, uint32_t n_out,
                                                uint32_t R, const int* rows, int nb,
                                                uint64_t b_addr, FoldOps& f) {
  const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(b_addr);
  const RLD_GLOBAL uint16_t* out = gp<const uint16_t>(out_addr);
  // The thread index passes through an empty asm: the fold's per-thread
  // offsets are then computed here, not hoisted to the kernel's start where
  // they would hold registers through the shrink.
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const bool kin = (uint32_t)(8 * lg) < R;  // this lane's 8 k of the 32-wide step hold rank
  if (ISSUE_B) {
#pragma unroll
    for (int t = 0; t < kFuseTiles; ++t) {
      const uint32_t col = (uint32_t)(wave * kFuseTiles + t) * 16u + cl;
      f.bt[t] = load16(B + (size_t)(col < n_out ? col : 0) * R + (kin ? 8 * lg : 0));
    }
  }
  if (ISSUE_BASE) {
#pragma unroll
    for (int j = 0; j < fold_pieces<FQ>(); ++j) {
      const int ei = tid + kGwThreads * j;
      const int rl = ei / (kFuseCols / 8);
      const uint32_t col = (uint32_t)(ei % (kFuseCols / 8)) * 8u;
      f.bv[j] = load16(out + (size_t)rows[rl < nb ? rl : 0] * os + (col < n_out ? col : 0u));
    }
  }
}

template <int FQ = 2>
__device__ __forceinline__ void wide_fold_finish(uint64_t out_addr, uint32_t os, uint32_t n_out,
                                                 uint32_t R, const int* rows, int nb,
                                                 float scale, FoldOps& f, const uint16_t* xl,
                                                 uint16_t* dl) {
  constexpr int QB = FQ;
  RLD_GLOBAL uint16_t* out = gp<uint16_t>(out_addr);
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const bool kin = (uint32_t)(8 * lg) < R;
  uint4 xf[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q)
    xf[q] = kin ? *reinterpret_cast<const uint4*>(&xl[(q * 16 + cl) * kXlStride + 8 * lg])
                : zero16();
  // k past max_rank and columns past n_out contribute nothing
#pragma unroll
  for (int t = 0; t < kFuseTiles; ++t) {
    const uint32_t col = (uint32_t)(wave * kFuseTiles + t) * 16u + cl;
    if (!kin || col >= n_out) f.bt[t] = zero16();
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if (q * 16 >= nb) continue;
#pragma unroll
    for (int t = 0; t < kFuseTiles; ++t) {
      const floatx4 acc = mfma_bf16_16x16x32(f.bt[t], xf[q], floatx4{0.f, 0.f, 0.f, 0.f});
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2*>(
          &dl[(q * 16 + cl) * kFuseStride + (wave * kFuseTiles + t) * 16 + 4 * lg]) =
          u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < fold_pieces<FQ>(); ++j) {
    const int ei = tid + kGwThreads * j;
    const int rl = ei / (kFuseCols / 8);
    const int c8 = (ei % (kFuseCols / 8)) * 8;
    const uint32_t col = (uint32_t)c8;
    if (rl < nb && col < n_out) {
      const uint4 dv = *reinterpret_cast<const uint4*>(&dl[rl * kFuseStride + c8]);
      store16(out + (size_t)rows[rl] * os + col, fold8(f.bv[j], dv, scale));
    }
  }
  __syncthreads();
}

// A projection of a wide launch: its xa and output, and the table entries the
// worklist kept in LDS.
struct WideProj {
  uint64_t xa_, out_;
  uint32_t os, n_out;
  const uint64_t* atab;
  const uint64_t* btab;
  const float* bscale;
};

// Item (pair, half h) of a wide launch over NP projections that share the
// routing (NP = 2: the pair kernel).  A projection that does not adapt the pair
// writes zero xa rows for the item's rows.
template <int NT, int PC, bool FUSE, int NP, int QB>
__device__ void gs_wide_item(const GsArgs& a, GsSmem<PC, kGwThreads>& sm,
                             floatx4 (*red)[QB * NT][kWave], int pair, int h,
                             const WideProj* pj, uint16_t* xl) {
  constexpr int KS = 4;   // MFMA steps per wave: 128 k
  constexpr int kRows = 16 * QB;
  const GroupedRows& g = a.gr;
  const uint32_t R = a.R, k_in = a.k_in;
  const int s = pair / (int)g.E;
  const int e = pair % (int)g.E;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t kw0 = (uint32_t)wave * (32u * KS);
  uint32_t lo, hi;
  span_in_window(sm.off, g, e, a.row_offset, a.row_end, lo, hi);
  const RLD_GLOBAL uint16_t* x = a.x();
  // The wave's k range lies inside k_in (every wave when k_in is a multiple of
  // 128): one pointer per operand row, the steps at immediate offsets.
  // Otherwise clamped in-bounds addresses, and k past k_in zeroed once loaded.
  const bool full = kw0 + 32u * KS <= k_in;
  // A_{s,e} over the wave's k range serves every batch of the item: the shrink
  // kernel issues it before the row scan, whose first wait covers it.  The
  // fused kernels load it with each batch's x rows instead, so that it is not
  // held through the fold (which needs those registers); only the merged path
  // of the pair kernel issues its first batch's tiles before the scan.
  uint4 bop[NT][KS];
  auto load_a_to = [&](uint4 (&dst)[NT][KS], const uint64_t* atab) {
    // the address is read from LDS at each call: computed once and kept, the
    // eight row addresses would hold registers through the fold
    // (the lane's offsets too, from a thread index laundered through an empty
    // asm, so that they are not hoisted to the kernel's start)
    const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(atab[pair]);
    int tl = (int)threadIdx.x;
    asm volatile("" : "+v"(tl));
    const int acl = tl & 15, alg = (tl >> 4) & 3;
    const uint32_t akw0 = (uint32_t)(tl >> 6) * (32u * KS);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t col = 16u * j + acl;
      const RLD_GLOBAL uint16_t* ar = A + (size_t)(col < R ? col : 0) * k_in;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kk = akw0 + 32u * ks + 8u * alg;
        dst[j][ks] = load16(full ? ar + kk : ar + (kk < k_in ? kk : 0));
      }
    }
  };
  auto mask_a_to = [&](uint4 (&dst)[NT][KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      if (kw0 + 32u * ks + 8u * lg >= k_in) {
#pragma unroll
        for (int j = 0; j < NT; ++j) dst[j][ks] = zero16();
      }
  };
  if (!FUSE) {
    load_a_to(bop, pj[0].atab);
    issue_point();
  }
  // MERGED: both projections of a pair kernel adapt the pair (a code path of
  // its own, so that the second projection's A tiles, which go out before the
  // row scan, hold registers only there)
  auto run = [&](auto merged_tag) {
    constexpr bool MERGED = decltype(merged_tag)::value;
    uint4 a1[MERGED ? NT : 1][KS];
    bool a_loaded = false;
    if constexpr (MERGED) {
      load_a_to(bop, pj[0].atab);
      load_a_to(a1, pj[NP - 1].atab);
      issue_point();
      a_loaded = true;
    }
    bool masked = full || FUSE;
    uint32_t c0 = lo;
    while (c0 < hi) {
      const int cnt = gs_scan(g, sm, e, s, &c0, hi, a.x_gather);
      if (!masked) {
        mask_a_to(bop);
        masked = true;
      }
      // half h takes its share of the scanned rows, ceil(cnt / 2) for h = 0
      const int split = (cnt + 1) / 2;
      const int bend = h ? cnt : split;
      for (int b0 = h ? split : 0; b0 < bend; b0 += kRows) {
        const int nb = min(bend - b0, kRows);
        // x fragments of 16-row subtile q (clamped rows past nb, k past k_in zeroed)
        auto load_x = [&](uint4 (&v)[KS], int q) {
          int tl = (int)threadIdx.x;  // laundered: the offsets are not hoisted
          asm volatile("" : "+v"(tl));
          const int li = q * 16 + (tl & 15);
          const uint32_t xk0 = (uint32_t)(tl >> 6) * (32u * KS) + 8u * ((tl >> 4) & 3);
          const RLD_GLOBAL uint16_t* xr = x + (size_t)sm.xrow[b0 + (li < nb ? li : 0)] * a.xs;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint32_t kk = xk0 + 32u * ks;
            v[ks] = load16(full ? xr + kk : xr + (kk < k_in ? kk : 0));
          }
        };
        auto mask_x = [&](uint4 (&v)[KS]) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            if (kw0 + 32u * ks + 8u * lg >= k_in) v[ks] = zero16();
        };
        // the wave's chain of subtile q, column tile j: its K steps in order
        auto chain = [&](const uint4 (&v)[KS], const uint4 (&w)[KS]) {
          floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16_16x16x32(v[ks], w[ks], acc);
          return acc;
        };
        auto mfma_x = [&](const uint4 (&v)[KS], int q) {
#pragma unroll
          for (int j = 0; j < NT; ++j) red[wave][q * NT + j][lane] = chain(v, bop[j]);
        };
        // one thread per (subtile, column tile, lane): the 16 wave sums in wave
        // order, rounded, to xl (fused) and the projection's xa rows (thread
        // index through an empty asm: the xa addresses are computed here)
        auto wave_sums = [&](const WideProj& P) {
          int ts = (int)threadIdx.x;
          asm volatile("" : "+v"(ts));
          if (ts < QB * NT * kWave && (ts / (NT * kWave)) * 16 < nb) {
            const int q = ts / (NT * kWave);
            const int j = (ts / kWave) % NT;
            const int ln = ts & 63;
            const uint32_t col = 16u * j + (ln & 15);
            floatx4 sum = red[0][q * NT + j][ln];
#pragma unroll
            for (int v = 1; v < kGwWaves; ++v) sum += red[v][q * NT + j][ln];
            if (col < R) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int li = q * 16 + 4 * (ln >> 4) + i;
                const uint16_t v = (uint16_t)f32_to_bf16(sum[i]);
                if (FUSE) xl[li * kXlStride + col] = v;
                if (li < nb) {
                  const uint32_t lr = (uint32_t)sm.list[b0 + li] - a.row_offset;
                  gp<uint16_t>(P.xa_)[(size_t)lr * R + col] = v;
                }
              }
            }
          }
        };
        // the fold of the batch's rows in one pass (the B tiles already issued
        // into f): up to 48 rows, whose delta tile (74.5 KB) fits the wave-sum
        // buffer; batches of up to 32 rows take the two-subtile form
        auto fold = [&](const WideProj& P, FoldOps& f) {
          uint16_t* dl = reinterpret_cast<uint16_t*>(&red[0][0][0]);
          if (QB > 2 && nb > 32) {
            wide_fold_issue<false, true, 3>(P.out_, P.os, P.n_out, R, sm.list + b0, nb,
                                            P.btab[pair], f);
            issue_point();
            wide_fold_finish<3>(P.out_, P.os, P.n_out, R, sm.list + b0, nb, P.bscale[pair], f, xl,
                                dl);
          } else {
            wide_fold_issue<false, true, 2>(P.out_, P.os, P.n_out, R, sm.list + b0, min(nb, 32),
                                            P.btab[pair], f);
            issue_point();
            wide_fold_finish<2>(P.out_, P.os, P.n_out, R, sm.list + b0, min(nb, 32), P.bscale[pair],
                                f, xl, dl);
          }
        };
        if constexpr (MERGED) {
          {
            // Both projections adapt the pair: one pass over the batch's x rows
            // runs the chains of both (each the chain the projection alone runs),
            // the first projection's go to the wave-sum buffer, the second's stay
            // in registers through the first one's sums and fold.
            floatx4 acc1[QB][NT];
            if (!a_loaded) {
              load_a_to(bop, pj[0].atab);
              load_a_to(a1, pj[1].atab);
            }
            a_loaded = false;
            auto mfma_both = [&](const uint4 (&v)[KS], int q) {
#pragma unroll
              for (int j = 0; j < NT; ++j) red[wave][q * NT + j][lane] = chain(v, bop[j]);
#pragma unroll
              for (int j = 0; j < NT; ++j) acc1[q][j] = chain(v, a1[j]);
            };
            // A third subtile (rows 32..47) goes out with the first two, but to
            // LDS (direct loads, no registers): each lane's four 16-byte
            // fragments land at lane * 16 in four 1 KB pieces of this wave's
            // wave-sum entries of subtiles 1 and 2 (4 KB at NT = 2), which are
            // written only after the pieces are read back.  At NT = 1 those
            // entries hold 2 KB: the third subtile is a second round of loads.
            const bool third = NT >= 2 && QB > 2 && nb > 32;
            auto stage_x2 = [&]() {
              static_assert(KS * kWave * 16 <= (QB * NT - NT) * kWave * (int)sizeof(floatx4) ||
                                NT < 2,
                            "the staged subtile fits the wave's entries of subtiles 1 and 2");
              int tl = (int)threadIdx.x;  // laundered: the offsets are not hoisted
              asm volatile("" : "+v"(tl));
              const int li = 32 + (tl & 15);
              const uint32_t xk0 = (uint32_t)(tl >> 6) * (32u * KS) + 8u * ((tl >> 4) & 3);
              const RLD_GLOBAL uint16_t* xr =
                  x + (size_t)sm.xrow[b0 + (li < nb ? li : 0)] * a.xs;
              unsigned char* st = reinterpret_cast<unsigned char*>(&red[wave][NT][0]);
#pragma unroll
              for (int ks = 0; ks < KS; ++ks) {
                const uint32_t kk = xk0 + 32u * ks;
                __builtin_amdgcn_global_load_lds(
                    (const void*)(full ? xr + kk : xr + (kk < k_in ? kk : 0)),
                    (__attribute__((address_space(3))) void*)(st + ks * kWave * 16), 16, 0, 0);
              }
            };
            {
              uint4 xq[2][KS];
              load_x(xq[0], 0);
              load_x(xq[1], 1);
              if (third) stage_x2();
              issue_point();
              if (!full) {
                mask_a_to(bop);
                mask_a_to(a1);
                mask_x(xq[0]);
                mask_x(xq[1]);
              }
              mfma_both(xq[0], 0);
              if (third) {
                // subtile 1's first-projection chains wait in registers while
                // the third subtile is read back from where they go
                floatx4 g1[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) g1[j] = chain(xq[1], bop[j]);
#pragma unroll
                for (int j = 0; j < NT; ++j) acc1[1][j] = chain(xq[1], a1[j]);
                uint4 x2[KS];
                const uint4* st = reinterpret_cast<const uint4*>(&red[wave][NT][0]);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) x2[ks] = st[ks * kWave + lane];
                if (!full) mask_x(x2);
#pragma unroll
                for (int j = 0; j < NT; ++j) red[wave][NT + j][lane] = g1[j];
                mfma_both(x2, 2);
              } else {
                mfma_both(xq[1], 1);
              }
            }
            if (NT < 2 && QB > 2 && nb > 32) {
              uint4 x2[KS];
              issue_point();  // not hoisted above the first subtiles' MFMAs
              load_x(x2, 2);
              issue_point();
              if (!full) mask_x(x2);
              mfma_both(x2, 2);
            }
            // the A tiles are dead until the next batch reloads them: constants
            // here, so that they hold no registers through the sums and folds
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
              for (int ks = 0; ks < KS; ++ks) bop[j][ks] = a1[j][ks] = zero16();
            FoldOps f0;
            issue_point();
            wide_fold_issue<true, false>(pj[0].out_, pj[0].os, pj[0].n_out, R, sm.list + b0,
                                         min(nb, 32), pj[0].btab[pair], f0);
            issue_point();
            __syncthreads();
            wave_sums(pj[0]);
            __syncthreads();
            fold(pj[0], f0);
            // the second projection: its chains to the (free again) buffer
#pragma unroll
            for (int q = 0; q < QB; ++q)
              if (q < 2 || nb > 32) {
#pragma unroll
                for (int j = 0; j < NT; ++j) red[wave][q * NT + j][lane] = acc1[q][j];
              }
            FoldOps f1;
            issue_point();
            wide_fold_issue<true, false>(pj[1].out_, pj[1].os, pj[1].n_out, R, sm.list + b0,
                                         min(nb, 32), pj[1].btab[pair], f1);
            issue_point();
            __syncthreads();
            wave_sums(pj[1]);
            __syncthreads();
            fold(pj[1], f1);
            continue;
          }
        } else {
#pragma unroll
        for (int pi = 0; pi < NP; ++pi) {
          const WideProj& P = pj[pi];
          if (NP > 1 && !((sm.valid[pair] >> pi) & 1)) {
            // this projection does not adapt the pair: zero xa rows (thread index
            // through an empty asm: these addresses are not hoisted out of the loops)
            int t0 = (int)threadIdx.x;
            asm volatile("" : "+v"(t0));
            for (int t = t0; t < nb * (int)(R / 8); t += kGwThreads)
              store16(gp<uint16_t>(P.xa_) +
                          (size_t)((uint32_t)sm.list[b0 + t / (int)(R / 8)] - a.row_offset) * R +
                          8 * (t % (int)(R / 8)),
                      zero16());
            continue;
          }
          if (FUSE) load_a_to(bop, P.atab);
          // Subtiles 0 and 1 go out with A; a third (rows 32..47 of the batch) is
          // a second round, with A still held, so that the common batch needs no
          // more registers than two subtiles.
          {
            uint4 aop[2][KS];
            load_x(aop[0], 0);
            load_x(aop[1], 1);
            issue_point();
            if (!full) {
              if (FUSE) mask_a_to(bop);
              mask_x(aop[0]);
              mask_x(aop[1]);
            }
            mfma_x(aop[0], 0);
            mfma_x(aop[1], 1);
          }
          if (QB > 2 && nb > 32) {
            uint4 x2[KS];
            load_x(x2, 2);
            issue_point();
            if (!full) mask_x(x2);
            mfma_x(x2, 2);
          }
          // the fold's B tiles go out now, so that their round trip overlaps
          // the wave sums
          FoldOps f0;
          issue_point();  // after the MFMAs' wave sums are stored
          if (FUSE)
            wide_fold_issue<true, false>(P.out_, P.os, P.n_out, R, sm.list + b0, min(nb, 32),
                                         P.btab[pair], f0);
          issue_point();
          __syncthreads();
          wave_sums(P);
          __syncthreads();
          if (FUSE) fold(P, f0);
        }
        }
      }
    }
  };
  if (NP > 1 && FUSE && (sm.valid[pair] & 3) == 3)
    run(std::integral_constant<bool, (NP > 1 && FUSE)>{});
  else
    run(std::integral_constant<bool, false>{});
}

// Items of the wide kernels: pair halves in groups of 8 pairs, then row blocks.
template <int NT, int PC, bool FUSE, int NP, int QB>
__device__ __forceinline__ void wide_items(const GsArgs& a, GsSmem<PC, kGwThreads>& sm,
                                           floatx4 (*red)[QB * NT][kWave], int na,
                                           const WideProj* pj, uint16_t* xl) {
  const uint32_t npi = 16u * (((uint32_t)na + 7u) / 8u);
  const uint32_t total = npi + a.nz;
  for (uint32_t it = blockIdx.x; it < total; it += gridDim.x) {
    if (it < npi) {
      const uint32_t p = (it / 16u) * 8u + it % 8u;
      if (p < (uint32_t)na)
        gs_wide_item<NT, PC, FUSE, NP, QB>(a, sm, red, sm.apairs[p], (int)((it / 8u) % 2u), pj,
                                           xl);
    } else {
      gs_zero_item(a, sm, it - npi, NP > 1 ? pj[1].xa_ : 0);
    }
  }
}

template <int NT, int PC>
__global__ __launch_bounds__(kGwThreads) void grouped_shrink_wide_kernel(GsArgs a) {
  __shared__ GsSmem<PC, kGwThreads> sm;
  __shared__ floatx4 red[kGwWaves][kWideQB * NT][kWave];
  PairKeep k0;
  k0.a = sm.atab;
  const int na = build_worklist<kGwThreads, PC, 1>(a.gr, a.row_offset, a.row_end, sm.off,
                                                   sm.valid, sm.apairs, sm.wcount, k0);
  WideProj pj[1];
  pj[0] = WideProj{a.xa_, 0, 0, 0, sm.atab, nullptr, nullptr};
  wide_items<NT, PC, false, 1, kWideQB>(a, sm, red, na, pj, nullptr);
}

// Shrink and fold of a window in one launch (rld_moe_grouped in the wide case);
// NP = 2 folds two projections that share the routing (rld_moe_grouped_pair),
// the second one's x rows read again from cache.  The wave-sum buffer doubles
// as the delta tile of the fold.
template <int NT, int PC, int NP>
__device__ __forceinline__ void fold_wide_body(const GsArgs& a) {
  constexpr int QB = kWideQB;
  constexpr size_t kRedBytes = sizeof(floatx4) * kGwWaves * QB * NT * kWave;
  constexpr size_t kDlBytes = sizeof(uint16_t) * 16 * QB * kFuseStride;  // a batch's delta tile
  __shared__ GsSmem<PC, kGwThreads> sm;
  __shared__ uint64_t btab[NP][PC];
  __shared__ float bscale[NP][PC];
  __shared__ uint64_t atab2[NP > 1 ? PC : 1];
  // xa of a batch (up to 64 rows of room), which the fold reads
  __shared__ __attribute__((aligned(16))) uint16_t xl[32 * ((QB + 1) / 2) * kXlStride];
  __shared__ __attribute__((aligned(16))) unsigned char buf[kRedBytes > kDlBytes ? kRedBytes
                                                                                : kDlBytes];
  auto red = reinterpret_cast<floatx4 (*)[QB * NT][kWave]>(buf);
  PairKeep k0, k1;
  k0.a = sm.atab;
  k0.b = btab[0];
  k0.scale = bscale[0];
  k0.scale_table = a.scale_table();
  if (NP > 1) {
    k1.a = atab2;
    k1.b = btab[NP - 1];
    k1.scale = bscale[NP - 1];
    k1.scale_table = gp<const float>(a.scale2_);
    k1.at = gp<const uint64_t>(a.atab2_);
    k1.bt = gp<const uint64_t>(a.btab2_);
  }
  const int na = build_worklist<kGwThreads, PC, 3, NP>(a.gr, a.row_offset, a.row_end, sm.off,
                                                       sm.valid, sm.apairs, sm.wcount, k0, k1);
  WideProj pj[NP];
  pj[0] = WideProj{a.xa_, a.out_, a.os, a.n_out, sm.atab, btab[0], bscale[0]};
  if (NP > 1)
    pj[NP - 1] = WideProj{a.xa2_, a.out2_, a.os2, a.n_out2, atab2, btab[NP - 1],
                          bscale[NP - 1]};
  wide_items<NT, PC, true, NP, QB>(a, sm, red, na, pj, xl);
}

template <int NT, int PC>
__global__ __launch_bounds__(kGwThreads) void grouped_fold_wide_kernel(GsArgs a) {
  fold_wide_body<NT, PC, 1>(a);
}

template <int NT, int PC>
__global__ __launch_bounds__(kGwThreads) void grouped_fold_pair_kernel(GsArgs a) {
  fold_wide_body<NT, PC, 2>(a);
}

// Item: (pair, 512 output columns).  The pair's B rows for the columns go to
// registers as MFMA A operands (each wave 64 columns); the pair's rows stream
// in batches of 64: their base values are prefetched, their xa rows are the B
// operand, deltas go to LDS as BF16 and are folded back in 16-byte pieces.
// NKS = ceil(max_rank / 32) K steps.
template <int NKS, int PC>
__global__ __launch_bounds__(kPeThreads) void grouped_expand_kernel(
    uint64_t xa_addr, GroupedRows gr, uint64_t scale_addr,
    uint32_t n_out, uint32_t R, uint32_t row_offset, uint32_t row_end, uint32_t nct,
    uint64_t out_addr, uint32_t os) {
  const RLD_GLOBAL uint16_t* xa = gp<const uint16_t>(xa_addr);
  const RLD_GLOBAL float* scale_table = gp<const float>(scale_addr);
  RLD_GLOBAL uint16_t* out = gp<uint16_t>(out_addr);
  __shared__ uint64_t btab[PC];
  __shared__ float bscale[PC];
  __shared__ int off_s[off_cap<PC>()];
  __shared__ uint8_t valid[PC];
  __shared__ int16_t apairs[PC];
  __shared__ int list[kListCap];
  __shared__ int toks[kListCap];
  __shared__ int wcount[kPeThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint16_t dl[kBatch * kDlStride];

  PairKeep k0;
  k0.b = btab;
  k0.scale = bscale;
  k0.scale_table = scale_table;
  const int na = build_worklist<kPeThreads, PC, 2>(gr, row_offset, row_end, off_s, valid, apairs,
                                                   wcount, k0);
  const int* off = off_s;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  constexpr int kFold = kBatch * (kPeCols / 8) / kPeThreads;  // uint4 per thread per batch

  for (int it = (int)blockIdx.x; it < na * (int)nct; it += (int)gridDim.x) {
    const int pair = apairs[it / (int)nct];
    const uint32_t j0 = (uint32_t)(it % (int)nct) * kPeCols;
    const int s = pair / (int)gr.E;
    const int e = pair % (int)gr.E;
    const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(btab[pair]);
    const float scale = bscale[pair];
    uint4 aop[4][NKS];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t c = j0 + wave * 64 + m * 16 + cl;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t k = ks * 32 + lg * 8;
        aop[m][ks] = load16(B + (c < n_out && k < R ? (size_t)c * R + k : 0));
        if (c >= n_out || k >= R) aop[m][ks] = zero16();
      }
    }
    uint32_t lo, hi;
    span_in_window(off, gr, e, row_offset, row_end, lo, hi);
    uint32_t c0 = lo;
    while (c0 < hi) {
      int cnt = 0;
      while (c0 < hi && cnt + (int)blockDim.x <= kListCap) {
        cnt += append_pair_rows(gr, off, e, s, c0, min(c0 + blockDim.x, hi), list, toks, cnt,
                                wcount);
        c0 += blockDim.x;
      }
      for (int b0 = 0; b0 < cnt; b0 += kBatch) {
        const int nb = min(cnt - b0, kBatch);
        uint4 bv[kFold];
#pragma unroll
        for (int j = 0; j < kFold; ++j) {
          const int ei = threadIdx.x + kPeThreads * j;
          const int rl = ei / (kPeCols / 8);
          const uint32_t c = j0 + (ei % (kPeCols / 8)) * 8;
          // clamped in-bounds address; entries past the batch or n_out are not stored
          bv[j] = load16(out + (size_t)list[b0 + (rl < nb ? rl : 0)] * os + (c < n_out ? c : j0));
        }
        // xa rows of the batch's four subtiles, all in flight with the base
        // values (clamped in-bounds addresses; k past max_rank zeroed)
        uint4 bop[kBatch / 16][NKS];
#pragma unroll
        for (int p = 0; p < kBatch / 16; ++p) {
          const int li = p * 16 + cl;
          const RLD_GLOBAL uint16_t* xr =
              xa + (size_t)((uint32_t)list[b0 + (li < nb ? li : 0)] - row_offset) * R;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint32_t k = ks * 32 + lg * 8;
            bop[p][ks] = load16(xr + (k < R ? k : 0));
          }
        }
        issue_point();
#pragma unroll
        for (int p = 0; p < kBatch / 16; ++p)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            if (ks * 32 + lg * 8 >= (int)R) bop[p][ks] = zero16();
#pragma unroll
        for (int p = 0; p < kBatch / 16; ++p) {
          if (p * 16 >= nb) continue;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16_16x16x32(aop[m][ks], bop[p][ks], acc);
            const uint32_t d01 = pack_bf16x2(acc[0], acc[1]);
            const uint32_t d23 = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<uint2*>(
                &dl[(p * 16 + cl) * kDlStride + wave * 64 + m * 16 + 4 * lg]) =
                make_uint2(d01, d23);
          }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kFold; ++j) {
          const int ei = threadIdx.x + kPeThreads * j;
          const int rl = ei / (kPeCols / 8);
          const int c8 = (ei % (kPeCols / 8)) * 8;
          const uint32_t c = j0 + c8;
          if (rl < nb && c < n_out) {
            const uint4 dv = *reinterpret_cast<const uint4*>(&dl[rl * kDlStride + c8]);
            store16(out + (size_t)list[b0 + rl] * os + c, fold8(bv[j], dv, scale));
          }
        }
        __syncthreads();
      }
    }
  }
}

static int check_grouped(const rld_moe_route* route, int x_gather, const int32_t* expert_offsets,
                         uint32_t num_experts_off, const int32_t* sorted_token_ids,
                         const int32_t* row_adapter, uint32_t row_offset, uint32_t row_end) {
  int st = check_moe_route(route);
  if (st) return st;
  if ((uint64_t)route->max_loras * route->num_experts > (uint64_t)kPairCapLarge)
    return RLD_EUNSUPPORTED;
  if (!expert_offsets || num_experts_off == 0) return RLD_EINVAL;
  if (num_experts_off >= (uint32_t)off_cap<kPairCapLarge>()) return RLD_EUNSUPPORTED;
  if (row_end < row_offset || row_end > 0x7fffffffu) return RLD_EINVAL;
  if ((x_gather || row_adapter) && !sorted_token_ids) return RLD_EINVAL;
  return RLD_OK;
}

// The route and offsets fit the small worklist instantiation.
static bool small_caps(const rld_moe_route* route, uint32_t num_experts_off) {
  return (uint64_t)route->max_loras * route->num_experts <= (uint64_t)kPairCapSmall &&
         num_experts_off < (uint32_t)off_cap<kPairCapSmall>();
}

// A row's token is read, and checked against num_tokens, whenever
// sorted_token_ids is given: the shrink (which may gather x by token), the
// expand (which never does) and the fused kernels then skip the same rows.
static GroupedRows make_rows(const rld_moe_route* route, uint32_t num_tokens,
                             const int32_t* expert_offsets, uint32_t num_experts_off,
                             const int32_t* sorted_token_ids, const int32_t* row_adapter) {
  GroupedRows g;
  g.off_ = reinterpret_cast<uint64_t>(expert_offsets);
  g.stid_ = reinterpret_cast<uint64_t>(sorted_token_ids);
  g.radapt_ = reinterpret_cast<uint64_t>(row_adapter);
  g.atab_ = reinterpret_cast<uint64_t>(route->a_table);
  g.btab_ = reinterpret_cast<uint64_t>(route->b_table);
  g.E_off = num_experts_off;
  g.num_tokens = num_tokens;
  g.max_loras = route->max_loras;
  g.E = route->num_experts;
  g.need_tok = sorted_token_ids ? 1 : 0;
  return g;
}

template <int KS, int NT, int PC>
static void launch_gs(const GsArgs& a, uint32_t grid, hipStream_t st) {
  hipLaunchKernelGGL((grouped_shrink_kernel<KS, NT, PC>), dim3(grid), dim3(kGsThreads), 0, st, a);
}

template <int KS, int PC>
static void launch_gs_nt(uint32_t nt, const GsArgs& a, uint32_t grid, hipStream_t st) {
  switch (nt) {
    case 1: launch_gs<KS, 1, PC>(a, grid, st); break;
    case 2: launch_gs<KS, 2, PC>(a, grid, st); break;
    default: launch_gs<KS, 4, PC>(a, grid, st); break;
  }
}

// KS = chunk / 128 (MFMA steps per wave), one of the chunk lengths grouped_chunk gives.
template <int PC>
static void launch_gs_ks(uint32_t ks, uint32_t nt, const GsArgs& a, uint32_t grid, hipStream_t st) {
  switch (ks) {
    case 2: launch_gs_nt<2, PC>(nt, a, grid, st); break;
    case 4: launch_gs_nt<4, PC>(nt, a, grid, st); break;
    case 6: launch_gs_nt<6, PC>(nt, a, grid, st); break;
    default: launch_gs_nt<8, PC>(nt, a, grid, st); break;
  }
}

}  // namespace rld

using namespace rld;

extern "C" size_t rld_moe_grouped_workspace_bytes(uint32_t window_rows, uint32_t k_in,
                                                  uint32_t max_rank, uint32_t max_loras,
                                                  uint32_t num_experts) {
  return grouped_workspace(window_rows, k_in, max_rank, max_loras, num_experts);
}

// The shrink of a window; with fold_out (rld_moe_grouped) in the wide case
// the fused kernel also folds the window into fold_out and *folded is set.
static int grouped_shrink(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                          int x_gather, uint32_t num_tokens, const int32_t* expert_offsets,
                          uint32_t num_experts_off, const int32_t* sorted_token_ids,
                          const int32_t* row_adapter, uint32_t row_offset, uint32_t row_end,
                          void* xa, uint32_t xa_rows_cap, void* workspace,
                          size_t workspace_bytes, void* stream, void* fold_out,
                          uint32_t fold_os, bool* folded) {
  *folded = false;
  int st = check_grouped(route, x_gather, expert_offsets, num_experts_off, sorted_token_ids,
                         row_adapter, row_offset, row_end);
  if (st) return st;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if (row_end - row_offset > xa_rows_cap) return RLD_ENOSPACE;
  if (row_end == row_offset) return RLD_OK;
  const uint32_t W = row_end - row_offset;
  const size_t need =
      grouped_workspace(W, route->k_in, route->max_rank, route->max_loras, route->num_experts);
  if (need) {
    if (!workspace) return RLD_EINVAL;
    if (!aligned16(workspace)) return RLD_EALIGN;
    if (workspace_bytes < need) return RLD_ENOSPACE;
  }
  GsArgs a = GsArgs{};
  a.x_ = reinterpret_cast<uint64_t>(x);
  a.xa_ = reinterpret_cast<uint64_t>(xa);
  a.part_ = reinterpret_cast<uint64_t>(workspace);
  a.ctr_ = reinterpret_cast<uint64_t>(workspace) + (workspace_bytes & ~(size_t)15);
  a.gr = make_rows(route, num_tokens, expert_offsets, num_experts_off,
                   sorted_token_ids, row_adapter);
  a.xs = x_row_stride;
  a.x_gather = x_gather ? 1u : 0u;
  a.k_in = route->k_in;
  a.R = route->max_rank;
  a.row_offset = row_offset;
  a.row_end = row_end;
  a.kc = grouped_chunk(route->k_in, route->max_rank);
  a.nch = div_ceil(route->k_in, a.kc);
  const uint32_t nt = grouped_nt(route->max_rank);
  a.ncg = div_ceil(div_ceil(route->max_rank, 16u), nt);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const uint64_t np = (uint64_t)route->max_loras * route->num_experts;
  if (grouped_wide(route->k_in, route->max_rank)) {
    a.nz = div_ceil(W, (uint32_t)kGwThreads);
    const uint64_t items = 16u * ((np + 7u) / 8u) + a.nz;
    const uint32_t grid = (uint32_t)(items < kGwGrid ? items : kGwGrid);
    const bool sm = small_caps(route, num_experts_off);
    auto kern = nt == 1 ? (sm ? grouped_shrink_wide_kernel<1, kPairCapSmall>
                              : grouped_shrink_wide_kernel<1, kPairCapLarge>)
                        : (sm ? grouped_shrink_wide_kernel<2, kPairCapSmall>
                              : grouped_shrink_wide_kernel<2, kPairCapLarge>);
    if (fold_out && route->n_out <= (uint32_t)kFuseCols) {
      a.out_ = reinterpret_cast<uint64_t>(fold_out);
      a.os = fold_os;
      a.n_out = route->n_out;
      a.scale_ = reinterpret_cast<uint64_t>(route->scale_table);
      kern = nt == 1 ? (sm ? grouped_fold_wide_kernel<1, kPairCapSmall>
                           : grouped_fold_wide_kernel<1, kPairCapLarge>)
                     : (sm ? grouped_fold_wide_kernel<2, kPairCapSmall>
                           : grouped_fold_wide_kernel<2, kPairCapLarge>);
      *folded = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGwThreads), 0, hs, a);
    return launch_status();
  }
  a.nz = div_ceil(W, (uint32_t)kGsThreads);
  // one chunk and one column group: (pair, row half) items (the kernel pairs
  // items it and it + 8 on one XCD, so the grid is a multiple of 8)
  const uint64_t items = (a.nch == 1 && a.ncg == 1 ? 16u * ((np + 7u) / 8u)
                                                   : np * a.nch * a.ncg) + a.nz;
  const uint64_t items8 = (items + 7u) & ~(uint64_t)7u;
  const uint32_t grid = (uint32_t)(items8 < kGsGrid ? items8 : kGsGrid);
  if (small_caps(route, num_experts_off))
    launch_gs_ks<kPairCapSmall>(a.kc / 128u, nt, a, grid, hs);
  else
    launch_gs_ks<kPairCapLarge>(a.kc / 128u, nt, a, grid, hs);
  return launch_status();
}

extern "C" int rld_moe_grouped_shrink(const rld_moe_route* route, const void* x,
                                      uint32_t x_row_stride, int x_gather, uint32_t num_tokens,
                                      const int32_t* expert_offsets, uint32_t num_experts_off,
                                      const int32_t* sorted_token_ids,
                                      const int32_t* row_adapter, uint32_t row_offset,
                                      uint32_t row_end, void* xa, uint32_t xa_rows_cap,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  bool folded;
  return grouped_shrink(route, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                        num_experts_off, sorted_token_ids, row_adapter, row_offset, row_end, xa,
                        xa_rows_cap, workspace, workspace_bytes, stream, nullptr, 0, &folded);
}

extern "C" int rld_moe_grouped_expand_fold(const rld_moe_route* route, const void* xa,
                                           uint32_t num_tokens, const int32_t* expert_offsets,
                                           uint32_t num_experts_off,
                                           const int32_t* sorted_token_ids,
                                           const int32_t* row_adapter, uint32_t row_offset,
                                           uint32_t row_end, void* base_out,
                                           uint32_t out_row_stride, void* stream) {
  int st = check_grouped(route, 0, expert_offsets, num_experts_off, sorted_token_ids,
                         row_adapter, row_offset, row_end);
  if (st) return st;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  if (row_end == row_offset) return RLD_OK;
  const uint32_t nct = div_ceil(route->n_out, kPeCols);
  GroupedRows gr = make_rows(route, num_tokens, expert_offsets, num_experts_off,
                             sorted_token_ids, row_adapter);
  const bool sm = small_caps(route, num_experts_off);
  auto kern = grouped_expand_kernel<1, kPairCapLarge>;
  switch (div_ceil(route->max_rank, 32)) {
    case 1: kern = sm ? grouped_expand_kernel<1, kPairCapSmall> : grouped_expand_kernel<1, kPairCapLarge>; break;
    case 2: kern = sm ? grouped_expand_kernel<2, kPairCapSmall> : grouped_expand_kernel<2, kPairCapLarge>; break;
    case 3: kern = sm ? grouped_expand_kernel<3, kPairCapSmall> : grouped_expand_kernel<3, kPairCapLarge>; break;
    default: kern = sm ? grouped_expand_kernel<4, kPairCapSmall> : grouped_expand_kernel<4, kPairCapLarge>; break;
  }
  hipLaunchKernelGGL(kern, dim3(kPeGrid), dim3(kPeThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<uint64_t>(xa), gr,
                     reinterpret_cast<uint64_t>(route->scale_table), route->n_out,
                     route->max_rank, row_offset, row_end, nct,
                     reinterpret_cast<uint64_t>(base_out), out_row_stride);
  return launch_status();
}

extern "C" int rld_moe_grouped(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                               int x_gather, uint32_t num_tokens, const int32_t* expert_offsets,
                               uint32_t num_experts_off, const int32_t* sorted_token_ids,
                               const int32_t* row_adapter, uint32_t row_offset, uint32_t row_end,
                               void* base_out, uint32_t out_row_stride, void* xa,
                               uint32_t xa_rows_cap, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int st = check_grouped(route, x_gather, expert_offsets, num_experts_off, sorted_token_ids,
                         row_adapter, row_offset, row_end);
  if (st) return st;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  bool folded = false;
  st = grouped_shrink(route, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                      num_experts_off, sorted_token_ids, row_adapter, row_offset, row_end, xa,
                      xa_rows_cap, workspace, workspace_bytes, stream, base_out, out_row_stride,
                      &folded);
  if (st || folded) return st;
  return rld_moe_grouped_expand_fold(route, xa, num_tokens, expert_offsets, num_experts_off,
                                     sorted_token_ids, row_adapter, row_offset, row_end,
                                     base_out, out_row_stride, stream);
}

extern "C" int rld_moe_grouped_pair(const rld_moe_route* route_a, const rld_moe_route* route_b,
                                    const void* x, uint32_t x_row_stride, int x_gather,
                                    uint32_t num_tokens, const int32_t* expert_offsets,
                                    uint32_t num_experts_off, const int32_t* sorted_token_ids,
                                    const int32_t* row_adapter, uint32_t row_offset,
                                    uint32_t row_end, void* base_a, uint32_t os_a, void* base_b,
                                    uint32_t os_b, void* xa_a, void* xa_b, uint32_t xa_rows_cap,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_grouped(route_a, x_gather, expert_offsets, num_experts_off, sorted_token_ids,
                         row_adapter, row_offset, row_end);
  if (st) return st;
  if ((st = check_grouped(route_b, x_gather, expert_offsets, num_experts_off, sorted_token_ids,
                          row_adapter, row_offset, row_end)))
    return st;
  if ((st = check_rows(x, x_row_stride, route_a->k_in))) return st;
  if ((st = check_rows(x, x_row_stride, route_b->k_in))) return st;
  if ((st = check_rows(base_a, os_a, route_a->n_out))) return st;
  if ((st = check_rows(base_b, os_b, route_b->n_out))) return st;
  if (!xa_a || !xa_b) return RLD_EINVAL;
  if (!aligned16(xa_a) || !aligned16(xa_b)) return RLD_EALIGN;
  if (row_end - row_offset > xa_rows_cap) return RLD_ENOSPACE;
  if (row_end == row_offset) return RLD_OK;
  const bool together = route_a->k_in == route_b->k_in &&
                        route_a->max_rank == route_b->max_rank &&
                        route_a->max_loras == route_b->max_loras &&
                        route_a->num_experts == route_b->num_experts &&
                        grouped_wide(route_a->k_in, route_a->max_rank) &&
                        route_a->n_out <= (uint32_t)kFuseCols &&
                        route_b->n_out <= (uint32_t)kFuseCols &&
                        small_caps(route_a, num_experts_off);  // LDS holds both routes' tables
  if (!together) {
    st = rld_moe_grouped(route_a, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                         num_experts_off, sorted_token_ids, row_adapter, row_offset, row_end,
                         base_a, os_a, xa_a, xa_rows_cap, workspace, workspace_bytes, stream);
    if (st) return st;
    return rld_moe_grouped(route_b, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                           num_experts_off, sorted_token_ids, row_adapter, row_offset, row_end,
                           base_b, os_b, xa_b, xa_rows_cap, workspace, workspace_bytes, stream);
  }
  const uint32_t W = row_end - row_offset;
  GsArgs a = GsArgs{};
  a.x_ = reinterpret_cast<uint64_t>(x);
  a.xa_ = reinterpret_cast<uint64_t>(xa_a);
  a.gr = make_rows(route_a, num_tokens, expert_offsets, num_experts_off,
                   sorted_token_ids, row_adapter);
  a.xs = x_row_stride;
  a.x_gather = x_gather ? 1u : 0u;
  a.k_in = route_a->k_in;
  a.R = route_a->max_rank;
  a.row_offset = row_offset;
  a.row_end = row_end;
  a.kc = grouped_chunk(a.k_in, a.R);
  a.nch = 1;
  a.ncg = 1;
  a.nz = div_ceil(W, (uint32_t)kGwThreads);
  a.out_ = reinterpret_cast<uint64_t>(base_a);
  a.os = os_a;
  a.n_out = route_a->n_out;
  a.scale_ = reinterpret_cast<uint64_t>(route_a->scale_table);
  a.xa2_ = reinterpret_cast<uint64_t>(xa_b);
  a.out2_ = reinterpret_cast<uint64_t>(base_b);
  a.os2 = os_b;
  a.n_out2 = route_b->n_out;
  a.scale2_ = reinterpret_cast<uint64_t>(route_b->scale_table);
  a.atab2_ = reinterpret_cast<uint64_t>(route_b->a_table);
  a.btab2_ = reinterpret_cast<uint64_t>(route_b->b_table);
  const uint64_t np = (uint64_t)route_a->max_loras * route_a->num_experts;
  const uint64_t items = 16u * ((np + 7u) / 8u) + a.nz;
  const uint32_t grid = (uint32_t)(items < kGwGrid ? items : kGwGrid);
  auto kern = grouped_nt(a.R) == 1 ? grouped_fold_pair_kernel<1, kPairCapSmall>
                                    : grouped_fold_pair_kernel<2, kPairCapSmall>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGwThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     a);
  return launch_status();
}
