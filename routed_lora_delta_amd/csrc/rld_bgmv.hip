// Routed BGMV ("Function apply_lora_bgmv"; lora_delta.rs, apply_lora_bgmv):
// every row i of a batch names an adapter slot s = seq_slot[i]; the shrink writes
// xa[i] = bf16(x_i @ A_s^T) and the expand folds bf16(xa[i] @ B_s^T), scaled in
// fp32 after the rounding, into the row's output.
//
// Work is slot-grouped: an item serves one slot and all rows that name it, so
// each slot's A_s / B_s tile is streamed from HBM once per call instead of once
// per row.  The row list of a slot is rebuilt by every item from seq_slot (no
// host read), in ascending row order.
//
//   shrink item  (slot, k_in chunk, 16 columns of xa).  Each of the four waves
//                owns every fourth 32-wide K step of the chunk and issues all
//                of its A fragments at once; x fragments of the next 16 rows
//                are in flight while the current ones multiply.  The waves'
//                partial sums are added in wave order.  With several chunks,
//                each item writes fp32 partials, and the item that finishes
//                the last chunk of a (slot, 16 columns) pair adds the chunks in
//                chunk order and writes xa (a counter per pair in the
//                workspace).  The chunk length depends only on (k_in,
//                max_rank), so a row's summation order is the same whatever
//                the batch holds: a batched call is bit-identical to one-row
//                calls.
//   expand item  (slot, 256 output columns).  B_s rows of the tile stay in
//                registers as MFMA A operands; rows of the slot stream through
//                as the B operand (16 rows per MFMA).  The base values of a
//                64-row pass are loaded before its MFMAs, deltas are rounded to
//                BF16 into LDS, and the fold writes 16-byte coalesced vectors.
//
// k-split partials move between blocks with agent-scope (L2-coherent across
// XCDs) stores and loads, and each block's stores have completed before it
// raises its group's counter, so no whole-cache writeback or invalidate is
// needed.  rld_bgmv launches the shrink, then the expand, on the caller's
// stream.
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

constexpr int kShrinkMT = 4;     // 16-row M-subtiles per shrink pass
constexpr int kShrinkSteps = 8;  // K steps per wave per chunk (chunk <= 1024 = 4 waves x 8 x 32)
constexpr int kListCap = 512;    // rows collected per pass over seq_slot
constexpr int kJT = 256;         // output columns per expand item
constexpr int kExpRows = 64;     // rows per fold pass of the expand
constexpr int kDlStride = kJT + 8;
constexpr int kFoldVecs = kExpRows * (kJT / 8) / 256;  // base vectors per thread per pass

static_assert(kShrinkSteps * 4 * 32 >= 1024, "a chunk is at most 1024 elements");

struct BgmvArgs {
  const uint16_t* x;
  const int32_t* seq_slot;
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  float* partial;  // [nch][n][R] fp32 (k split only), at the start of the workspace
  uint32_t* book;  // end of the workspace: slot s's 8 chunk counters (one per
                   // 16-column group of xa) are the 8 words at book - 8 (s + 1)
  uint16_t* xa;
  uint16_t* out;
  uint32_t xs, n, max_loras, k_in, n_out, R, kc, nch, ntr, os;
};

struct ShrinkSmem {
  int rows[kListCap];
  int wcount[4];
  floatx4 red[4][kShrinkMT][kWave];
  int flag;
};

struct ExpandSmem {
  int rows[kListCap];
  int wcount[4];
  __attribute__((aligned(16))) uint16_t dl[kExpRows * kDlStride];
};

__device__ __forceinline__ uint32_t* slot_counters(const BgmvArgs& a, int s) {
  return a.book - 8 * ((size_t)s + 1);
}

__device__ __forceinline__ bool slot_active(const BgmvArgs& a, int s) {
  return s >= 0 && (uint32_t)s < a.max_loras && a.a_table[s] != 0ull && a.b_table[s] != 0ull;
}

// Appends to `rows` (LDS) the rows of slot s from seq_slot[*pos ...], until
// n is reached or the list cannot take another 256; advances *pos.  Returns
// the count (the same in every thread).
__device__ __forceinline__ int collect_slot_rows(const int32_t* __restrict__ seq_slot, uint32_t n,
                                                 uint32_t* pos, int s, int* rows, int* wcount) {
  int cnt = 0;
  while (*pos < n && cnt <= kListCap - 256) {
    cnt += append_matching_rows(seq_slot, n, *pos, s, rows, cnt, wcount);
    *pos += 256;
  }
  return cnt;
}

// Block-wide: this thread's stores have completed, then the block meets, then
// thread 0 adds 1 to *ctr (agent scope) and every thread gets the old value.
__device__ __forceinline__ uint32_t block_signal(uint32_t* ctr, int* slot) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *slot = (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t old = (uint32_t)*slot;
  __syncthreads();
  return old;
}

// Shrink item w (slot-major over (slot, chunk, 16 columns)).
__device__ void shrink_item(const BgmvArgs& a, uint32_t w, ShrinkSmem& sm) {
  const uint32_t n = a.n, R = a.R, nchunks = a.nch, ntr = a.ntr;
  const uint32_t rt = w % ntr;
  const uint32_t c = (w / ntr) % nchunks;
  const int s = (int)(w / (ntr * nchunks));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // The first item also writes the zero xa rows of base rows.
  if (w == 0) {
    const uint32_t r8 = R / 8;
    for (uint32_t e = threadIdx.x; e < n * r8; e += 256) {
      const uint32_t row = e / r8;
      if (!slot_active(a, a.seq_slot[row]))
        *reinterpret_cast<uint4*>(a.xa + (size_t)row * R + (e % r8) * 8) = zero16();
    }
  }
  if (!slot_active(a, s)) return;

  const uint16_t* A = reinterpret_cast<const uint16_t*>(a.a_table[s]);
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t col = rt * 16 + cl;  // xa column = A_s row served by this lane
  const bool col_ok = col < R;
  const uint16_t* Arow = A + (size_t)(col_ok ? col : 0) * a.k_in;
  const uint32_t kb = c * a.kc;
  const uint32_t ke = min(kb + a.kc, a.k_in);
  const uint32_t nsteps = (ke - kb + 31) / 32;

  // This wave's K steps are wave, wave + 4, ...: all of its A fragments are
  // issued here, before the row scan waits on seq_slot.
  uint4 bop[kShrinkSteps];
  uint32_t kof[kShrinkSteps];
  bool kok[kShrinkSteps];
#pragma unroll
  for (int i = 0; i < kShrinkSteps; ++i) {
    const uint32_t st = wave + 4 * i;
    kof[i] = kb + st * 32 + lg * 8;
    kok[i] = st < nsteps && kof[i] < ke;
    bop[i] = (col_ok && kok[i]) ? load16(Arow + kof[i]) : zero16();
  }

  uint32_t pos = 0;
  int first_row = -1;
  int scans = 0, last_cnt = 0;
  while (pos < n) {
    const int cnt = collect_slot_rows(a.seq_slot, n, &pos, s, sm.rows, sm.wcount);
    ++scans;
    last_cnt = cnt;
    if (first_row < 0 && cnt > 0) first_row = sm.rows[0];
    for (int b0 = 0; b0 < cnt; b0 += kShrinkMT * 16) {
      const int nb = min(cnt - b0, kShrinkMT * 16);
      const int nmt = (nb + 15) >> 4;
      floatx4 acc[kShrinkMT];
#pragma unroll
      for (int q = 0; q < kShrinkMT; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
      // x fragments of subtile q + 1 are issued before the MFMAs of subtile q
      uint4 cur[kShrinkSteps], nxt[kShrinkSteps];
#pragma unroll
      for (int i = 0; i < kShrinkSteps; ++i) nxt[i] = zero16();
      {
        const bool ok = cl < nb;
        const uint16_t* xr = a.x + (size_t)(ok ? sm.rows[b0 + cl] : 0) * a.xs;
#pragma unroll
        for (int i = 0; i < kShrinkSteps; ++i)
          cur[i] = (ok && kok[i]) ? load16(xr + kof[i]) : zero16();
      }
#pragma unroll
      for (int q = 0; q < kShrinkMT; ++q) {
        if (q < nmt) {
          if (q + 1 < nmt) {
            const int li = (q + 1) * 16 + cl;
            const bool ok = li < nb;
            const uint16_t* xr = a.x + (size_t)(ok ? sm.rows[b0 + li] : 0) * a.xs;
#pragma unroll
            for (int i = 0; i < kShrinkSteps; ++i)
              nxt[i] = (ok && kok[i]) ? load16(xr + kof[i]) : zero16();
          }
#pragma unroll
          for (int i = 0; i < kShrinkSteps; ++i)
            acc[q] = mfma_bf16_16x16x32(cur[i], bop[i], acc[q]);
#pragma unroll
          for (int i = 0; i < kShrinkSteps; ++i) cur[i] = nxt[i];
        }
      }
#pragma unroll
      for (int q = 0; q < kShrinkMT; ++q)
        if (q < nmt) sm.red[wave][q][lane] = acc[q];
      __syncthreads();
      for (int q = wave; q < nmt; q += 4) {
        floatx4 sum = sm.red[0][q][lane];
        sum += sm.red[1][q][lane];
        sum += sm.red[2][q][lane];
        sum += sm.red[3][q][lane];
        if (col_ok) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int li = q * 16 + 4 * lg + i;
            if (li < nb) {
              const uint32_t row = (uint32_t)sm.rows[b0 + li];
              if (nchunks == 1) {
                a.xa[(size_t)row * R + col] = (uint16_t)f32_to_bf16(sum[i]);
              } else {  // agent-scope store: written through to where every XCD reads it
                __hip_atomic_store(a.partial + ((size_t)c * n + row) * R + col, sum[i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }
  if (first_row < 0 || nchunks == 1) return;

  // k split: the item that completes the last chunk of its (slot, 16 xa
  // columns) adds the chunks in chunk order and writes xa.  The group's
  // counter is left at zero.
  uint32_t* ctr = slot_counters(a, s) + rt;
  if (block_signal(ctr, &sm.flag) != nchunks - 1) return;
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const int rl = threadIdx.x >> 4;  // 16 rows x 16 columns per step
  const uint32_t rcol = rt * 16 + (threadIdx.x & 15);
  uint32_t rpos = 0;
  for (int batch = 0;; ++batch) {
    int cnt;
    if (scans == 1) {  // rows[] still holds the slot's whole list
      if (batch > 0) break;
      cnt = last_cnt;
    } else {
      if (rpos >= n) break;
      cnt = collect_slot_rows(a.seq_slot, n, &rpos, s, sm.rows, sm.wcount);
    }
    if (rcol < R) {
      for (int li = rl; li < cnt; li += 16) {
        const uint32_t row = (uint32_t)sm.rows[li];
        float* pp = a.partial + (size_t)row * R + rcol;
        const size_t cstride = (size_t)n * R;
        float sum = 0.f;
        for (uint32_t c0 = 0; c0 < nchunks; c0 += 8) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            v[j] = (c0 + j < nchunks) ? __hip_atomic_load(pp + (c0 + j) * cstride, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT)
                                      : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + j < nchunks) sum = (c0 + j == 0) ? v[j] : sum + v[j];
        }
        a.xa[(size_t)row * R + rcol] = (uint16_t)f32_to_bf16(sum);
      }
    }
    __syncthreads();
  }
}

// Expand item (slot s, 256 output columns from j0).  NKS = ceil(max_rank/32).
template <int NKS>
__device__ void expand_item(const BgmvArgs& a, int s, uint32_t j0, ExpandSmem& sm) {
  if (!slot_active(a, s)) return;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(a.b_table[s]);
  const float scale = a.scale_table[s];
  const uint32_t n = a.n, R = a.R, n_out = a.n_out, os = a.os;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;

  // B_s rows of this wave's 64 columns, as MFMA A operands for every K step.
  uint4 aop[4][NKS];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t col = j0 + wave * 64 + m * 16 + cl;
    const bool ok = col < n_out;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t k = ks * 32 + lg * 8;
      aop[m][ks] = (ok && k < R) ? load16(B + (size_t)col * R + k) : zero16();
    }
  }

  // fold mapping: vector i of a thread is row (tid / 32) + 8 i, columns c8 .. c8+7
  const int frow = threadIdx.x >> 5;
  const int c8 = (threadIdx.x & 31) * 8;
  const bool fcol_ok = j0 + c8 < n_out;

  uint32_t pos = 0;
  while (pos < n) {
    const int cnt = collect_slot_rows(a.seq_slot, n, &pos, s, sm.rows, sm.wcount);
    for (int b0 = 0; b0 < cnt; b0 += kExpRows) {
      const int nb = min(cnt - b0, kExpRows);
      // base values of the pass, issued before the MFMAs
      uint4 bv[kFoldVecs];
#pragma unroll
      for (int i = 0; i < kFoldVecs; ++i) {
        const int rl = frow + 8 * i;
        bv[i] = (rl < nb && fcol_ok)
                    ? *reinterpret_cast<const uint4*>(a.out + (size_t)sm.rows[b0 + rl] * os + j0 + c8)
                    : zero16();
      }
      uint4 bop[4][NKS];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int li = p * 16 + cl;
        const bool ok = li < nb;
        const uint16_t* xr = a.xa + (size_t)(ok ? sm.rows[b0 + li] : 0) * R;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint32_t k = ks * 32 + lg * 8;
          bop[p][ks] = (p * 16 < nb && ok && k < R) ? load16(xr + k) : zero16();
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p * 16 < nb) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16_16x16x32(aop[m][ks], bop[p][ks], acc);
            // lane holds delta[row p*16+cl][cols m*16 + 4*lg .. +3] of this wave's slice
            const uint32_t d01 = pack_bf16x2(acc[0], acc[1]);
            const uint32_t d23 = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<uint2*>(&sm.dl[(p * 16 + cl) * kDlStride + wave * 64 + m * 16 +
                                             4 * lg]) = make_uint2(d01, d23);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kFoldVecs; ++i) {
        const int rl = frow + 8 * i;
        if (rl < nb && fcol_ok) {
          const uint4 dv = *reinterpret_cast<const uint4*>(&sm.dl[rl * kDlStride + c8]);
          *reinterpret_cast<uint4*>(a.out + (size_t)sm.rows[b0 + rl] * os + j0 + c8) =
              fold8(bv[i], dv, scale);
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void bgmv_shrink_kernel(BgmvArgs a, uint32_t total) {
  __shared__ ShrinkSmem sm;
  // the ntr items of one (slot, chunk) share an XCD, and so the x rows in its L2
  const uint32_t w = xcd_group_item(a.ntr);
  if (w >= total) return;
  shrink_item(a, w, sm);
}

template <int NKS>
__global__ __launch_bounds__(256) void bgmv_expand_kernel(BgmvArgs a) {
  __shared__ ExpandSmem sm;
  expand_item<NKS>(a, (int)blockIdx.y, blockIdx.x * kJT, sm);
}

// Workspace: fp32 partials [nch][n][R] from the start (k split only), and at
// the end of the caller's buffer (its size rounded down to 16 bytes) 8 chunk
// counters per slot.  Keying the counters to the end of the buffer and to
// slots keeps them in one place for every call that shares the buffer,
// whatever their shapes.  They must be zero before the first call and are zero
// after every call.
static size_t round16(size_t v) { return (v + 15) & ~(size_t)15; }

static size_t partial_bytes(uint32_t n, uint32_t k_in, uint32_t R) {
  const uint32_t nch = div_ceil(k_in, bgmv_chunk(k_in, R));
  return nch > 1 ? round16((size_t)nch * n * R * sizeof(float)) : 0;
}

static size_t book_bytes(uint32_t max_loras) { return (size_t)max_loras * 32; }

static int make_args(const rld_route* route, const void* x, uint32_t x_row_stride,
                     const int32_t* seq_slot, uint32_t n, void* xa, void* workspace,
                     size_t workspace_bytes, void* base_out, uint32_t out_row_stride,
                     BgmvArgs* a) {
  const uint32_t R = route->max_rank, k_in = route->k_in;
  const size_t end = workspace_bytes & ~(size_t)15;
  if (!workspace || end < partial_bytes(n, k_in, R) + book_bytes(route->max_loras))
    return RLD_ENOSPACE;
  if (!aligned16(workspace)) return RLD_EALIGN;
  char* ws = static_cast<char*>(workspace);
  a->x = static_cast<const uint16_t*>(x);
  a->seq_slot = seq_slot;
  a->a_table = route->a_table;
  a->b_table = route->b_table;
  a->scale_table = route->scale_table;
  a->partial = reinterpret_cast<float*>(ws);
  a->book = reinterpret_cast<uint32_t*>(ws + end);
  a->xa = static_cast<uint16_t*>(xa);
  a->out = static_cast<uint16_t*>(base_out);
  a->xs = x_row_stride;
  a->n = n;
  a->max_loras = route->max_loras;
  a->k_in = k_in;
  a->n_out = route->n_out;
  a->R = R;
  a->kc = bgmv_chunk(k_in, R);
  a->nch = div_ceil(k_in, a->kc);
  a->ntr = div_ceil(R, 16);
  a->os = out_row_stride;
  return RLD_OK;
}

typedef void (*BgmvKernel)(BgmvArgs);

static BgmvKernel pick_expand(uint32_t R) {
  switch (div_ceil(R, 32)) {
    case 1: return bgmv_expand_kernel<1>;
    case 2: return bgmv_expand_kernel<2>;
    case 3: return bgmv_expand_kernel<3>;
    default: return bgmv_expand_kernel<4>;
  }
}

}  // namespace rld

using namespace rld;

extern "C" size_t rld_bgmv_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank,
                                           uint32_t max_loras) {
  if (k_in == 0 || max_rank == 0 || max_loras == 0) return 0;
  return partial_bytes(n, k_in, max_rank) + book_bytes(max_loras);
}

extern "C" int rld_bgmv_shrink(const rld_route* route, const void* x, uint32_t x_row_stride,
                               const int32_t* seq_slot, uint32_t n, void* xa, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (route->max_loras > 65535u) return RLD_EUNSUPPORTED;
  if (n == 0) return RLD_OK;
  if (!seq_slot || !xa) return RLD_EINVAL;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!aligned16(xa)) return RLD_EALIGN;
  BgmvArgs a;
  if ((st = make_args(route, x, x_row_stride, seq_slot, n, xa, workspace, workspace_bytes,
                      nullptr, 0, &a)))
    return st;
  const uint32_t total = route->max_loras * a.nch * a.ntr;
  hipLaunchKernelGGL(bgmv_shrink_kernel, dim3(xcd_group_grid(total, a.ntr)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), a, total);
  return launch_status();
}

extern "C" int rld_bgmv_expand_fold(const rld_route* route, const void* xa,
                                    const int32_t* seq_slot, uint32_t n, void* base_out,
                                    uint32_t out_row_stride, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (route->max_loras > 65535u) return RLD_EUNSUPPORTED;
  if (n == 0) return RLD_OK;
  if (!seq_slot || !xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  BgmvArgs a = {};
  a.seq_slot = seq_slot;
  a.a_table = route->a_table;
  a.b_table = route->b_table;
  a.scale_table = route->scale_table;
  a.xa = const_cast<uint16_t*>(static_cast<const uint16_t*>(xa));
  a.out = static_cast<uint16_t*>(base_out);
  a.n = n;
  a.max_loras = route->max_loras;
  a.k_in = route->k_in;
  a.n_out = route->n_out;
  a.R = route->max_rank;
  a.ntr = div_ceil(a.R, 16);
  a.os = out_row_stride;
  hipLaunchKernelGGL(pick_expand(a.R), dim3(div_ceil(route->n_out, kJT), route->max_loras),
                     dim3(256), 0, reinterpret_cast<hipStream_t>(stream), a);
  return launch_status();
}

extern "C" int rld_bgmv(const rld_route* route, const void* x, uint32_t x_row_stride,
                        const int32_t* seq_slot, uint32_t n, void* base_out,
                        uint32_t out_row_stride, void* xa, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (n == 0) return RLD_OK;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  st = rld_bgmv_shrink(route, x, x_row_stride, seq_slot, n, xa, workspace, workspace_bytes,
                       stream);
  if (st) return st;
  return rld_bgmv_expand_fold(route, xa, seq_slot, n, base_out, out_row_stride, stream);
}
