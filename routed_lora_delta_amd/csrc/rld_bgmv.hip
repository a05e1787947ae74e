// Routed BGMV ("Function apply_lora_bgmv"; lora_delta.rs, apply_lora_bgmv):
// every row i of a batch names an adapter slot s = seq_slot[i]; the shrink writes
// xa[i] = bf16(x_i @ A_s^T) and the expand folds bf16(xa[i] @ B_s^T), scaled in
// fp32 after the rounding, into the row's output.
//
// Kernels are slot-grouped: a block serves one slot and all rows that name it,
// so each slot's A_s / B_s tile is streamed from HBM once per call instead of
// once per row.  The row list of a slot is rebuilt in every block from
// seq_slot (no host read), in ascending row order.
//
//   shrink  block = (slot, k_in chunk, 16 columns of xa).  Each of the four
//           waves owns every fourth 32-wide K step of the chunk and issues all
//           of its A fragments at once; x fragments of the next 16 rows are in
//           flight while the current ones multiply.  The waves' partial sums
//           are added in wave order.  With several chunks, each block writes
//           fp32 partials, and the block that finishes the last chunk of a
//           (slot, 16 columns) pair adds the chunks in chunk order and writes
//           xa (a counter per pair in the workspace; no second launch).  The
//           chunk length depends only on (k_in, max_rank), so a row's
//           summation order is the same whatever the batch holds: a batched
//           call is bit-identical to one-row calls.
//   expand  block = (slot, 256 output columns).  B_s rows of the tile stay in
//           registers as MFMA A operands; rows of the slot stream through as
//           the B operand (16 rows per MFMA).  The base values of a 64-row pass
//           are loaded before its MFMAs, deltas are rounded to BF16 into LDS,
//           and the fold writes 16-byte coalesced vectors.
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

constexpr int kShrinkMT = 4;     // 16-row M-subtiles per shrink pass
constexpr int kShrinkSteps = 8;  // K steps per wave per chunk (chunk <= 1024 = 4 waves x 8 x 32)
constexpr int kListCap = 512;    // rows collected per pass over seq_slot
constexpr int kJT = 256;         // output columns per expand block
constexpr int kExpRows = 64;     // rows per fold pass of the expand
constexpr int kDlStride = kJT + 8;
constexpr int kFoldVecs = kExpRows * (kJT / 8) / 256;  // base vectors per thread per pass

static_assert(kShrinkSteps * 4 * 32 >= 1024, "a chunk is at most 1024 elements");

__device__ __forceinline__ bool slot_active(const uint64_t* __restrict__ a_table,
                                            const uint64_t* __restrict__ b_table,
                                            uint32_t max_loras, int s) {
  return s >= 0 && (uint32_t)s < max_loras && a_table[s] != 0ull && b_table[s] != 0ull;
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

__global__ __launch_bounds__(256) void bgmv_shrink_kernel(
    const uint16_t* __restrict__ x, uint32_t xs, const int32_t* __restrict__ seq_slot, uint32_t n,
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    uint32_t max_loras, uint32_t k_in, uint32_t R, uint32_t kc, uint32_t nchunks, uint32_t ntr,
    uint32_t total, float* __restrict__ partial, uint32_t* __restrict__ counters,
    uint16_t* __restrict__ xa) {
  __shared__ int rows[kListCap];
  __shared__ int wcount[4];
  __shared__ floatx4 red[4][kShrinkMT][kWave];
  __shared__ int last_flag;

  // the ntr items of one (slot, chunk) share an XCD, and so the x rows in its L2
  const uint32_t w = xcd_group_item(ntr);
  if (w >= total) return;
  const uint32_t rt = w % ntr;
  const uint32_t c = (w / ntr) % nchunks;
  const int s = (int)(w / (ntr * nchunks));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // The first work item also writes the zero xa rows of base rows.
  if (w == 0) {
    const uint32_t r8 = R / 8;
    for (uint32_t e = threadIdx.x; e < n * r8; e += 256) {
      const uint32_t row = e / r8;
      if (!slot_active(a_table, b_table, max_loras, seq_slot[row]))
        *reinterpret_cast<uint4*>(xa + (size_t)row * R + (e % r8) * 8) = zero16();
    }
  }
  if (!slot_active(a_table, b_table, max_loras, s)) return;

  const uint16_t* A = reinterpret_cast<const uint16_t*>(a_table[s]);
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t col = rt * 16 + cl;  // xa column = A_s row served by this lane
  const bool col_ok = col < R;
  const uint16_t* Arow = A + (size_t)(col_ok ? col : 0) * k_in;
  const uint32_t kb = c * kc;
  const uint32_t ke = min(kb + kc, k_in);
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
    const int cnt = collect_slot_rows(seq_slot, n, &pos, s, rows, wcount);
    ++scans;
    last_cnt = cnt;
    if (first_row < 0 && cnt > 0) first_row = rows[0];
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
        const uint16_t* xr = x + (size_t)(ok ? rows[b0 + cl] : 0) * xs;
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
            const uint16_t* xr = x + (size_t)(ok ? rows[b0 + li] : 0) * xs;
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
        if (q < nmt) red[wave][q][lane] = acc[q];
      __syncthreads();
      for (int q = wave; q < nmt; q += 4) {
        floatx4 sum = red[0][q][lane];
        sum += red[1][q][lane];
        sum += red[2][q][lane];
        sum += red[3][q][lane];
        if (col_ok) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int li = q * 16 + 4 * lg + i;
            if (li < nb) {
              const uint32_t row = (uint32_t)rows[b0 + li];
              if (nchunks == 1)
                xa[(size_t)row * R + col] = (uint16_t)f32_to_bf16(sum[i]);
              else  // agent-scope store: written through to where every XCD reads it
                __hip_atomic_store(partial + ((size_t)c * n + row) * R + col, sum[i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
      __syncthreads();
    }
  }
  if (nchunks == 1 || first_row < 0) return;

  // k split: the block that completes the last chunk of its (slot, 16 xa
  // columns) adds the chunks in chunk order and writes xa.  The pair's counter
  // is keyed by the slot's first row (unique per slot) and is left at zero.
  // Partials travel with agent-scope (L2-coherent) stores and loads, and each
  // thread's stores have completed before the block's counter increment, so no
  // whole-cache writeback or invalidate is needed.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* ctr = counters + (size_t)first_row * ntr + rt;
  if (threadIdx.x == 0)
    last_flag = (__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 nchunks - 1) ? 1 : 0;
  __syncthreads();
  if (!last_flag) return;
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
      cnt = collect_slot_rows(seq_slot, n, &rpos, s, rows, wcount);
    }
    if (rcol < R) {
      for (int li = rl; li < cnt; li += 16) {
        const uint32_t row = (uint32_t)rows[li];
        float* pp = partial + (size_t)row * R + rcol;
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
        xa[(size_t)row * R + rcol] = (uint16_t)f32_to_bf16(sum);
      }
    }
    __syncthreads();
  }
}

template <int NKS>
__global__ __launch_bounds__(256) void bgmv_expand_kernel(
    const uint16_t* __restrict__ xa, const int32_t* __restrict__ seq_slot, uint32_t n,
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    const float* __restrict__ scale_table, uint32_t max_loras, uint32_t n_out, uint32_t R,
    uint16_t* __restrict__ out, uint32_t os) {
  __shared__ int rows[kListCap];
  __shared__ int wcount[4];
  __shared__ __attribute__((aligned(16))) uint16_t dl[kExpRows * kDlStride];

  const int s = (int)blockIdx.y;
  if (!slot_active(a_table, b_table, max_loras, s)) return;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(b_table[s]);
  const float scale = scale_table[s];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t j0 = blockIdx.x * kJT;

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
    const int cnt = collect_slot_rows(seq_slot, n, &pos, s, rows, wcount);
    for (int b0 = 0; b0 < cnt; b0 += kExpRows) {
      const int nb = min(cnt - b0, kExpRows);
      // base values of the pass, issued before the MFMAs
      uint4 bv[kFoldVecs];
#pragma unroll
      for (int i = 0; i < kFoldVecs; ++i) {
        const int rl = frow + 8 * i;
        bv[i] = (rl < nb && fcol_ok)
                    ? *reinterpret_cast<const uint4*>(out + (size_t)rows[b0 + rl] * os + j0 + c8)
                    : zero16();
      }
      uint4 bop[4][NKS];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int li = p * 16 + cl;
        const bool ok = li < nb;
        const uint16_t* xr = xa + (size_t)(ok ? rows[b0 + li] : 0) * R;
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
            *reinterpret_cast<uint2*>(&dl[(p * 16 + cl) * kDlStride + wave * 64 + m * 16 +
                                          4 * lg]) = make_uint2(d01, d23);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kFoldVecs; ++i) {
        const int rl = frow + 8 * i;
        if (rl < nb && fcol_ok) {
          const uint4 dv = *reinterpret_cast<const uint4*>(&dl[rl * kDlStride + c8]);
          *reinterpret_cast<uint4*>(out + (size_t)rows[b0 + rl] * os + j0 + c8) =
              fold8(bv[i], dv, scale);
        }
      }
      __syncthreads();
    }
  }
}

// Workspace layout of a k-split shrink: fp32 partials [chunks][n][max_rank],
// then one uint32 counter per (row, 16 xa columns).
static size_t partial_bytes(uint32_t n, uint32_t nch, uint32_t R) {
  return (size_t)nch * n * R * sizeof(float);
}

}  // namespace rld

using namespace rld;

extern "C" size_t rld_bgmv_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank) {
  if (k_in == 0 || max_rank == 0) return 0;
  const uint32_t nch = div_ceil(k_in, bgmv_chunk(k_in, max_rank));
  if (nch <= 1) return 0;
  const size_t ctr = (size_t)n * div_ceil(max_rank, 16) * sizeof(uint32_t);
  return partial_bytes(n, nch, max_rank) + ((ctr + 15) & ~(size_t)15);
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
  const uint32_t R = route->max_rank, k_in = route->k_in;
  const uint32_t kc = bgmv_chunk(k_in, R);
  const uint32_t nch = div_ceil(k_in, kc);
  const uint32_t ntr = div_ceil(R, 16);
  const size_t need = rld_bgmv_workspace_bytes(n, k_in, R);
  if (need > 0 && (!workspace || workspace_bytes < need)) return RLD_ENOSPACE;
  if (need > 0 && !aligned16(workspace)) return RLD_EALIGN;
  float* partial = static_cast<float*>(workspace);
  uint32_t* counters =
      need > 0 ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                             partial_bytes(n, nch, R))
               : nullptr;
  const uint32_t total = route->max_loras * nch * ntr;
  hipLaunchKernelGGL(bgmv_shrink_kernel, dim3(xcd_group_grid(total, ntr)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                     x_row_stride, seq_slot, n, route->a_table, route->b_table, route->max_loras,
                     k_in, R, kc, nch, ntr, total, partial, counters, static_cast<uint16_t*>(xa));
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
  auto kern = bgmv_expand_kernel<1>;
  switch (div_ceil(route->max_rank, 32)) {
    case 1: kern = bgmv_expand_kernel<1>; break;
    case 2: kern = bgmv_expand_kernel<2>; break;
    case 3: kern = bgmv_expand_kernel<3>; break;
    default: kern = bgmv_expand_kernel<4>; break;
  }
  hipLaunchKernelGGL(kern, dim3(div_ceil(route->n_out, kJT), route->max_loras), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint16_t*>(xa),
                     seq_slot, n, route->a_table, route->b_table, route->scale_table,
                     route->max_loras, route->n_out, route->max_rank,
                     static_cast<uint16_t*>(base_out), out_row_stride);
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
