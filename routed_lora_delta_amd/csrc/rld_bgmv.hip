// Routed BGMV ("Function apply_lora_bgmv"; lora_delta.rs, apply_lora_bgmv):
// every row i of a batch names an adapter slot s = seq_slot[i]; the shrink writes
// xa[i] = bf16(x_i @ A_s^T) and the expand folds bf16(xa[i] @ B_s^T), scaled in
// fp32 after the rounding, into the row's output.
//
// Kernels are slot-grouped: a block serves one slot and all rows that name it,
// so each slot's A_s / B_s tile is streamed from HBM once per call instead of
// once per row.  The row list of a slot is rebuilt in every block from
// seq_slot (no host read, no workspace), in ascending row order.
//
//   shrink  block = (slot, k_in chunk, 16 columns of xa).  The four waves share
//           the chunk's 32-wide K steps; their partial sums are added in wave
//           order, and chunks are added in chunk order by the reduce kernel.
//           The chunk length depends only on (k_in, max_rank), so a row's
//           summation order is the same whatever the batch holds: a batched
//           call is bit-identical to one-row calls.
//   expand  block = (slot, 256 output columns).  B_s rows of the tile stay in
//           registers as MFMA A operands; rows of the slot stream through as
//           the B operand (16 rows per MFMA).  Deltas are rounded to BF16 into
//           LDS, then folded into base_out with 16-byte coalesced accesses.
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

constexpr int kShrinkMT = 8;     // 16-row M-subtiles per shrink pass
constexpr int kListCap = 512;    // rows collected per pass over seq_slot
constexpr int kJT = 256;         // output columns per expand block
constexpr int kExpRows = 64;     // rows per fold pass of the expand
constexpr int kDlStride = kJT + 8;

__device__ __forceinline__ bool slot_active(const uint64_t* __restrict__ a_table,
                                            const uint64_t* __restrict__ b_table,
                                            uint32_t max_loras, int s) {
  return s >= 0 && (uint32_t)s < max_loras && a_table[s] != 0ull && b_table[s] != 0ull;
}

__global__ __launch_bounds__(256) void bgmv_shrink_kernel(
    const uint16_t* __restrict__ x, uint32_t xs, const int32_t* __restrict__ seq_slot, uint32_t n,
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    uint32_t max_loras, uint32_t k_in, uint32_t R, uint32_t kc, uint32_t nchunks, uint32_t ntr,
    uint32_t total, float* __restrict__ partial, uint16_t* __restrict__ xa) {
  __shared__ int rows[kListCap];
  __shared__ int wcount[4];
  __shared__ floatx4 red[4][kShrinkMT][kWave];

  const uint32_t w = xcd_work_item(total);
  if (w >= total) return;
  const uint32_t rt = w % ntr;
  const uint32_t c = (w / ntr) % nchunks;
  const int s = (int)(w / (ntr * nchunks));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // Single-chunk split writes xa directly; the first work item also writes the
  // zero xa rows of base rows (the reduce kernel does it otherwise).
  if (nchunks == 1 && w == 0) {
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

  uint32_t pos = 0;
  while (pos < n) {
    int cnt = 0;
    while (pos < n && cnt <= kListCap - 256) {
      cnt += append_matching_rows(seq_slot, n, pos, s, rows, cnt, wcount);
      pos += 256;
    }
    for (int b0 = 0; b0 < cnt; b0 += kShrinkMT * 16) {
      const int nb = min(cnt - b0, kShrinkMT * 16);
      const int nmt = (nb + 15) >> 4;
      const uint16_t* xr[kShrinkMT];
      bool xok[kShrinkMT];
#pragma unroll
      for (int q = 0; q < kShrinkMT; ++q) {
        const int li = q * 16 + cl;
        xok[q] = li < nb;
        xr[q] = x + (size_t)(xok[q] ? rows[b0 + li] : 0) * xs;
      }
      floatx4 acc[kShrinkMT];
#pragma unroll
      for (int q = 0; q < kShrinkMT; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (uint32_t st = wave; st < nsteps; st += 4) {
        const uint32_t k = kb + st * 32 + lg * 8;
        const bool kok = k < ke;
        const uint4 bop = (col_ok && kok) ? load16(Arow + k) : zero16();
#pragma unroll
        for (int q = 0; q < kShrinkMT; ++q) {
          if (q < nmt) {
            const uint4 aop = (xok[q] && kok) ? load16(xr[q] + k) : zero16();
            acc[q] = mfma_bf16_16x16x32(aop, bop, acc[q]);
          }
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
              else
                partial[((size_t)c * n + row) * R + col] = sum[i];
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

// xa[row, col] = bf16(sum over chunks c = 0, 1, ... of partial[c, row, col]);
// zero rows for base rows.
__global__ __launch_bounds__(256) void bgmv_reduce_kernel(
    const float* __restrict__ partial, const int32_t* __restrict__ seq_slot, uint32_t n,
    const uint64_t* __restrict__ a_table, const uint64_t* __restrict__ b_table,
    uint32_t max_loras, uint32_t R, uint32_t nchunks, uint16_t* __restrict__ xa) {
  const uint32_t idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * R) return;
  const uint32_t row = idx / R;
  uint32_t v = 0;
  if (slot_active(a_table, b_table, max_loras, seq_slot[row])) {
    float sum = partial[idx];
    for (uint32_t c = 1; c < nchunks; ++c) sum += partial[(size_t)c * n * R + idx];
    v = f32_to_bf16(sum);
  }
  xa[idx] = (uint16_t)v;
}

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
  const int nks = (int)((R + 31) / 32);

  // B_s rows of this wave's 64 columns, as MFMA A operands for every K step.
  uint4 aop[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t col = j0 + wave * 64 + m * 16 + cl;
    const bool ok = col < n_out;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t k = ks * 32 + lg * 8;
      aop[m][ks] = (ks < nks && ok && k < R) ? load16(B + (size_t)col * R + k) : zero16();
    }
  }

  uint32_t pos = 0;
  while (pos < n) {
    int cnt = 0;
    while (pos < n && cnt <= kListCap - 256) {
      cnt += append_matching_rows(seq_slot, n, pos, s, rows, cnt, wcount);
      pos += 256;
    }
    for (int b0 = 0; b0 < cnt; b0 += kExpRows) {
      const int nb = min(cnt - b0, kExpRows);
#pragma unroll
      for (int p = 0; p < kExpRows / 16; ++p) {
        if (p * 16 < nb) {
          const int li = p * 16 + cl;
          const bool ok = li < nb;
          const uint16_t* xr = xa + (size_t)(ok ? rows[b0 + li] : 0) * R;
          uint4 bop[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const uint32_t k = ks * 32 + lg * 8;
            bop[ks] = (ks < nks && ok && k < R) ? load16(xr + k) : zero16();
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              if (ks < nks) acc = mfma_bf16_16x16x32(aop[m][ks], bop[ks], acc);
            // lane holds delta[row p*16+cl][cols m*16 + 4*lg .. +3] of this wave's slice
            const uint32_t d01 = pack_bf16x2(acc[0], acc[1]);
            const uint32_t d23 = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<uint2*>(&dl[(p * 16 + cl) * kDlStride + wave * 64 + m * 16 +
                                          4 * lg]) = make_uint2(d01, d23);
          }
        }
      }
      __syncthreads();
      for (int e = threadIdx.x; e < nb * (kJT / 8); e += 256) {
        const int rl = e / (kJT / 8);
        const int c8 = (e % (kJT / 8)) * 8;
        const uint32_t col = j0 + c8;
        if (col < n_out) {
          uint16_t* p = out + (size_t)rows[b0 + rl] * os + col;
          const uint4 bv = *reinterpret_cast<const uint4*>(p);
          const uint4 dv = *reinterpret_cast<const uint4*>(&dl[rl * kDlStride + c8]);
          *reinterpret_cast<uint4*>(p) = fold8(bv, dv, scale);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace rld

using namespace rld;

extern "C" size_t rld_bgmv_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank) {
  if (k_in == 0 || max_rank == 0) return 0;
  const uint32_t nch = div_ceil(k_in, bgmv_chunk(k_in, max_rank));
  return nch > 1 ? (size_t)nch * n * max_rank * sizeof(float) : 0;
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
  const uint32_t total = route->max_loras * nch * ntr;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(bgmv_shrink_kernel, dim3(xcd_grid(total)), dim3(256), 0, sm,
                     static_cast<const uint16_t*>(x), x_row_stride, seq_slot, n, route->a_table,
                     route->b_table, route->max_loras, k_in, R, kc, nch, ntr, total,
                     static_cast<float*>(workspace), static_cast<uint16_t*>(xa));
  if ((st = launch_status())) return st;
  if (nch > 1) {
    hipLaunchKernelGGL(bgmv_reduce_kernel, dim3(div_ceil(n * R, 256)), dim3(256), 0, sm,
                       static_cast<const float*>(workspace), seq_slot, n, route->a_table,
                       route->b_table, route->max_loras, R, nch, static_cast<uint16_t*>(xa));
    st = launch_status();
  }
  return st;
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
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(bgmv_expand_kernel, dim3(div_ceil(route->n_out, kJT), route->max_loras),
                     dim3(256), 0, sm, static_cast<const uint16_t*>(xa), seq_slot, n,
                     route->a_table, route->b_table, route->scale_table, route->max_loras,
                     route->n_out, route->max_rank, static_cast<uint16_t*>(base_out),
                     out_row_stride);
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
