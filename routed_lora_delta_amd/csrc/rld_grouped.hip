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
// s, and streams A_{s,e} (shrink) or a column slice of B_{s,e} (expand) exactly
// once for all of them.  Every x row and every base row is touched by the one
// item of its pair, and the MFMA jobs are as tall as the pair's row count.
// Launches are persistent: a fixed number of blocks (host constant, so a
// captured launch keeps its shape), each of which lists the window's active
// pairs (adapter present, rows in the window) from the offsets and the tables
// in one round of loads, then takes its share of the items.  No block is spent
// on a pair that has nothing to do.
//
// Summation order.  The shrink splits k_in into 8 fixed ranges, one per wave
// (range length a function of k_in only); each wave sums its range in one MFMA
// chain, the 8 partial sums are added in wave order.  The expand is one MFMA
// chain over max_rank.  A row's result therefore never depends on which other
// rows share its block or window: a full-window call and the union of chunk
// windows are bit-identical.
//
// xa rows of window rows that do not fold are written as zeros, expert by
// expert (items after the pair items), and by block 0 for rows that no expert
// of the table owns.
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

constexpr int kOffCap = 1024;    // expert_offsets entries staged in LDS (num_experts_off < kOffCap)
constexpr int kPairCap = 2048;   // max_loras * num_experts held in the LDS worklist
constexpr int kListCap = 512;    // rows of a pair collected per scan
constexpr int kBatch = 64;       // rows of a pair per MFMA pass (4 subtiles of 16)
constexpr int kPsThreads = 512;  // shrink block: 8 waves, one k_in range each
constexpr int kPsWaves = kPsThreads / kWave;
constexpr int kPsSplit = 1;      // shrink blocks per pair (row subtiles split between them)
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

// All threads: expert_offsets into LDS (the launchers require E_off < kOffCap).
__device__ __forceinline__ const int* stage_offsets(const GroupedRows& g, int* off_s) {
  for (uint32_t i = threadIdx.x; i <= g.E_off; i += blockDim.x) off_s[i] = g.off()[i];
  __syncthreads();
  return off_s;
}

// Window part [lo, hi) of expert e's span (empty when e has no offsets entry).
__device__ __forceinline__ void span_in_window(const int* off, const GroupedRows& g, int e,
                                               uint32_t row_offset, uint32_t row_end,
                                               uint32_t& lo, uint32_t& hi) {
  lo = hi = row_end;
  if ((uint32_t)e >= g.E_off) return;
  const int64_t a = off[e], b = off[e + 1];
  lo = (uint32_t)max<int64_t>(a, row_offset);
  hi = (uint32_t)min<int64_t>(b, row_end);
  if (hi < lo) hi = lo;
}

// Adapter slot of sorted row r (slot 0 without row_adapter), or -1 when its
// token is out of range; the token goes to *tok.
__device__ __forceinline__ int row_slot(const GroupedRows& g, uint32_t r, int* tok) {
  int t = 0;
  if (g.need_tok) {
    t = g.stid()[r];
    if (t < 0 || (uint32_t)t >= g.num_tokens) return -1;
  }
  *tok = t;
  return g.radapt_ ? g.radapt()[t] : 0;
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
  for (uint32_t i = 0; i < R / 8; ++i) store16(xa + (size_t)local_row * R + 8 * i, zero16());
}

// Every thread: stage expert_offsets, read the A/B table entries of every pair
// (valid[p] = both present), and list in LDS, ascending, the pairs that are
// valid and own rows of [row_offset, row_end).  The offsets and table reads go
// out together, so this costs one round of loads.  Returns the pair count.
__device__ __forceinline__ int build_worklist(const GroupedRows& g, uint32_t row_offset,
                                              uint32_t row_end, int* off_s, uint8_t* valid,
                                              int16_t* apairs, int* wcount) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t np = g.max_loras * g.E;
  for (uint32_t i = threadIdx.x; i <= g.E_off; i += blockDim.x) off_s[i] = g.off()[i];
  for (uint32_t p = threadIdx.x; p < np; p += blockDim.x) {
    const uint64_t ta = g.a_table()[p], tb = g.b_table()[p];
    valid[p] = (ta != 0ull && tb != 0ull) ? 1 : 0;
  }
  __syncthreads();
  const int* off = off_s;
  int na = 0;
  for (uint32_t c0 = 0; c0 < np; c0 += blockDim.x) {
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

// Block = (pair (s, e), part h of kPsSplit).  Part h takes the 16-row subtiles
// q of the pair's row list with q % kPsSplit == h, so a pair's rows spread over
// kPsSplit blocks (placed on one XCD, where they share A_{s,e} in L2).  Wave
// w sums k_in range [w*kw, (w+1)*kw) for up to 4 subtiles at a time, loading
// that range of A once per pass and of each x row once; the 8 partial sums
// meet in LDS in wave order.
__global__ __launch_bounds__(kPsThreads) void grouped_shrink_kernel(
    uint64_t x_addr, uint32_t xs, int x_gather, GroupedRows gr, uint32_t k_in, uint32_t R,
    uint32_t row_offset, uint32_t row_end, uint32_t kw, uint32_t total, uint64_t xa_addr) {
  const RLD_GLOBAL uint16_t* x = gp<const uint16_t>(x_addr);
  RLD_GLOBAL uint16_t* xa = gp<uint16_t>(xa_addr);
  __shared__ int off_s[kOffCap];
  __shared__ int list[kListCap];
  __shared__ int toks[kListCap];
  __shared__ int wcount[kPsWaves];
  __shared__ floatx4 red[kPsWaves][8][kWave];

  const uint32_t w = xcd_work_item(total);
  if (w >= total) return;
  const int pair = (int)(w / kPsSplit);
  const int h = (int)(w % kPsSplit);
  const int s = pair / (int)gr.E;
  const int e = pair % (int)gr.E;
  const uint64_t ta = gr.a_table()[pair], tb = gr.b_table()[pair];  // with the offsets
  const int* off = stage_offsets(gr, off_s);
  const bool pair_ok = ta != 0ull && tb != 0ull;
  uint32_t lo, hi;
  span_in_window(off, gr, e, row_offset, row_end, lo, hi);

  if (s == 0 && h == 0) {
    // rows of e's span that no pair folds
    for (uint32_t r = lo + threadIdx.x; r < hi; r += blockDim.x) {
      if (expert_of_row(off, (int)gr.E_off, (int)r) != e) continue;
      int t = 0;
      const int sr = row_slot(gr, r, &t);
      bool act = sr >= 0 && (uint32_t)sr < gr.max_loras;
      if (act) {
        const int pr = sr * (int)gr.E + e;
        const uint64_t pa = gr.a_table()[pr], pb = gr.b_table()[pr];
        act = pa != 0ull && pb != 0ull;
      }
      if (!act) zero_xa_row(xa, r - row_offset, R);
    }
    if (e == 0) {
      // rows that no expert of the table owns
      for (uint32_t r = row_offset + threadIdx.x; r < row_end; r += blockDim.x) {
        const int o = expert_of_row(off, (int)gr.E_off, (int)r);
        if (o < 0 || (uint32_t)o >= gr.E) zero_xa_row(xa, r - row_offset, R);
      }
    }
  }
  if (!pair_ok || hi <= lo) return;

  const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(ta);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t kb = min(wave * kw, k_in);
  const uint32_t ke = min(kb + kw, k_in);
  const int ntn = (int)((R + 15) / 16);

  uint32_t c0 = lo;
  while (c0 < hi) {
    int cnt = 0;
    while (c0 < hi && cnt + (int)blockDim.x <= kListCap) {
      cnt += append_pair_rows(gr, off, e, s, c0, min(c0 + blockDim.x, hi), list, toks, cnt,
                              wcount);
      c0 += blockDim.x;
    }
    // this block's subtiles: q = h, h + kPsSplit, ... of the (cnt+15)/16
    const int nsub = (cnt + 15) >> 4;
    for (int q0 = h; q0 < nsub; q0 += 4 * kPsSplit) {
      const RLD_GLOBAL uint16_t* xr[4];
      bool rok[4];
      int nq = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qs = q0 + q * kPsSplit;
        nq += qs < nsub ? 1 : 0;
        const int li = qs * 16 + cl;
        rok[q] = qs < nsub && li < cnt;
        const int src = rok[q] ? (x_gather ? toks[li] : list[li]) : 0;
        xr[q] = x + (size_t)src * xs;
      }
      for (int n0 = 0; n0 < ntn; n0 += 2) {
        floatx4 acc[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[q][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (uint32_t k = kb; k < ke; k += 256) {
          uint4 bop[2][8];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t col = (n0 + j) * 16 + cl;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
              const uint32_t kk = k + ks * 32 + lg * 8;
              bop[j][ks] = (col < R && kk < ke) ? load16(A + (size_t)col * k_in + kk) : zero16();
            }
          }
          // x rows of the four subtiles: two in flight ahead of the MFMAs
          uint4 aop[4][8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q < 2) {
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                const uint32_t kk = k + ks * 32 + lg * 8;
                aop[q][ks] = (q < nq && rok[q] && kk < ke) ? load16(xr[q] + kk) : zero16();
              }
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q + 2 < 4) {
#pragma unroll
              for (int ks = 0; ks < 8; ++ks) {
                const uint32_t kk = k + ks * 32 + lg * 8;
                aop[q + 2][ks] =
                    (q + 2 < nq && rok[q + 2] && kk < ke) ? load16(xr[q + 2] + kk) : zero16();
              }
            }
            if (q < nq) {
#pragma unroll
              for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                  acc[q][j] = mfma_bf16_16x16x32(aop[q][ks], bop[j][ks], acc[q][j]);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 2; ++j) red[wave][q * 2 + j][lane] = acc[q][j];
        __syncthreads();
        {
          // one thread per (subtile, column tile, lane): partial sums in wave order
          const int q = threadIdx.x >> 7;
          const int j = (threadIdx.x >> 6) & 1;
          const int ln = threadIdx.x & 63;
          const uint32_t col = (n0 + j) * 16 + (ln & 15);
          if (q < nq && col < R) {
            floatx4 sum = red[0][q * 2 + j][ln];
#pragma unroll
            for (int v = 1; v < kPsWaves; ++v) sum += red[v][q * 2 + j][ln];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int li = (q0 + q * kPsSplit) * 16 + 4 * (ln >> 4) + i;
              if (li < cnt)
                xa[(size_t)((uint32_t)list[li] - row_offset) * R + col] =
                    (uint16_t)f32_to_bf16(sum[i]);
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

// Item: (pair, 512 output columns).  The pair's B rows for the columns go to
// registers as MFMA A operands (each wave 64 columns); the pair's rows stream
// in batches of 64: their base values are prefetched, their xa rows are the B
// operand, deltas go to LDS as BF16 and are folded back in 16-byte pieces.
// NKS = ceil(max_rank / 32) K steps.
template <int NKS>
__global__ __launch_bounds__(kPeThreads) void grouped_expand_kernel(
    uint64_t xa_addr, GroupedRows gr, uint64_t scale_addr,
    uint32_t n_out, uint32_t R, uint32_t row_offset, uint32_t row_end, uint32_t nct,
    uint64_t out_addr, uint32_t os) {
  const RLD_GLOBAL uint16_t* xa = gp<const uint16_t>(xa_addr);
  const RLD_GLOBAL float* scale_table = gp<const float>(scale_addr);
  RLD_GLOBAL uint16_t* out = gp<uint16_t>(out_addr);
  __shared__ int off_s[kOffCap];
  __shared__ uint8_t valid[kPairCap];
  __shared__ int16_t apairs[kPairCap];
  __shared__ int list[kListCap];
  __shared__ int toks[kListCap];
  __shared__ int wcount[kPeThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint16_t dl[kBatch * kDlStride];

  const int na = build_worklist(gr, row_offset, row_end, off_s, valid, apairs, wcount);
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
    const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(gr.b_table()[pair]);
    const float scale = scale_table[pair];
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
  if ((uint64_t)route->max_loras * route->num_experts > (uint64_t)kPairCap) return RLD_EUNSUPPORTED;
  if (!expert_offsets || num_experts_off == 0) return RLD_EINVAL;
  if (num_experts_off >= (uint32_t)kOffCap) return RLD_EUNSUPPORTED;
  if (row_end < row_offset || row_end > 0x7fffffffu) return RLD_EINVAL;
  if ((x_gather || row_adapter) && !sorted_token_ids) return RLD_EINVAL;
  return RLD_OK;
}

static GroupedRows make_rows(const rld_moe_route* route, int x_gather, uint32_t num_tokens,
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
  g.need_tok = (x_gather || row_adapter) ? 1 : 0;
  return g;
}

// Length of the k_in range of one shrink wave: the 8 ranges cover k_in, in
// multiples of 32.  A function of k_in only.
static uint32_t shrink_range(uint32_t k_in) { return 32u * div_ceil(k_in, 32u * kPsWaves); }

}  // namespace rld

using namespace rld;

extern "C" int rld_moe_grouped_shrink(const rld_moe_route* route, const void* x,
                                      uint32_t x_row_stride, int x_gather, uint32_t num_tokens,
                                      const int32_t* expert_offsets, uint32_t num_experts_off,
                                      const int32_t* sorted_token_ids,
                                      const int32_t* row_adapter, uint32_t row_offset,
                                      uint32_t row_end, void* xa, uint32_t xa_rows_cap,
                                      void* stream) {
  int st = check_grouped(route, x_gather, expert_offsets, num_experts_off, sorted_token_ids,
                         row_adapter, row_offset, row_end);
  if (st) return st;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if (row_end - row_offset > xa_rows_cap) return RLD_ENOSPACE;
  if (row_end == row_offset) return RLD_OK;
  GroupedRows gr = make_rows(route, x_gather, num_tokens, expert_offsets, num_experts_off,
                             sorted_token_ids, row_adapter);
  const uint32_t total = route->max_loras * route->num_experts * kPsSplit;
  hipLaunchKernelGGL(grouped_shrink_kernel, dim3(xcd_grid(total)), dim3(kPsThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<uint64_t>(x),
                     x_row_stride, x_gather ? 1 : 0, gr, route->k_in, route->max_rank,
                     row_offset, row_end, shrink_range(route->k_in), total,
                     reinterpret_cast<uint64_t>(xa));
  return launch_status();
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
  GroupedRows gr = make_rows(route, 0, num_tokens, expert_offsets, num_experts_off,
                             sorted_token_ids, row_adapter);
  auto kern = grouped_expand_kernel<1>;
  switch (div_ceil(route->max_rank, 32)) {
    case 1: kern = grouped_expand_kernel<1>; break;
    case 2: kern = grouped_expand_kernel<2>; break;
    case 3: kern = grouped_expand_kernel<3>; break;
    default: kern = grouped_expand_kernel<4>; break;
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
                               uint32_t xa_rows_cap, void* stream) {
  int st = check_grouped(route, x_gather, expert_offsets, num_experts_off, sorted_token_ids,
                         row_adapter, row_offset, row_end);
  if (st) return st;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  st = rld_moe_grouped_shrink(route, x, x_row_stride, x_gather, num_tokens, expert_offsets,
                              num_experts_off, sorted_token_ids, row_adapter, row_offset,
                              row_end, xa, xa_rows_cap, stream);
  if (st) return st;
  return rld_moe_grouped_expand_fold(route, xa, num_tokens, expert_offsets, num_experts_off,
                                     sorted_token_ids, row_adapter, row_offset, row_end,
                                     base_out, out_row_stride, stream);
}
