// MoE variants of the routed fold ("Module moe_lora_grouped").
//
// Gather fold (moe_lora_gather_bgmv): unsorted flat (token, top-k) rows; row rho
// takes its expert from indices[rho] and its adapter slot from
// row_adapter[rho / top_k].  Distinct (slot, expert) pairs rarely repeat across
// the rows of a decode step, so each row is a pair of GEMVs on the vector ALUs:
//   shrink  one block per row; each wave owns xa columns, its lanes split k_in
//           in 16-byte pieces and the partial sums meet in a fixed xor-butterfly.
//   expand  one block per (row, 512 columns); a thread owns two adjacent output
//           columns, sums over max_rank in order, and folds 4 bytes of base_out.
//
// Grouped fold (moe_lora_grouped_down): expert-sorted rows of one chunk window,
// in 64-row m-tiles.  A tile's rows are classified on the device (expert from
// the expert_offsets prefix sum, token from sorted_token_ids, slot from
// row_adapter) and grouped by (slot, expert) pair; every group is a small dense
// contraction on the matrix cores with that pair's A or B.
//   shrink  block = (m-tile, 16 xa columns); work units are (group, 16 rows),
//           each summing the whole k_in in one MFMA chain.
//   expand  block = (m-tile, 256 output columns); per group, B rows stay in
//           registers and the group's xa rows stream as the B operand; deltas
//           go to LDS as BF16 and are folded into base_out in 16-byte pieces.
// A row's result depends only on its own data and its pair, so a full-window
// call and the union of chunk windows are bit-identical.
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

constexpr int kJT = 256;
constexpr int kDlStride = kJT + 8;

// ------------------------------------------------------------------ gather --

__device__ __forceinline__ int gather_pair(uint32_t rho, const int32_t* __restrict__ indices,
                                           const int32_t* __restrict__ row_adapter,
                                           uint32_t top_k, const uint64_t* __restrict__ a_table,
                                           const uint64_t* __restrict__ b_table,
                                           uint32_t max_loras, uint32_t E) {
  const int s = row_adapter ? row_adapter[rho / top_k] : 0;
  const int e = indices[rho];
  if (s < 0 || (uint32_t)s >= max_loras || e < 0 || (uint32_t)e >= E) return -1;
  const int pair = s * (int)E + e;
  if (a_table[pair] == 0ull || b_table[pair] == 0ull) return -1;
  return pair;
}

// acc += sum_i a[i] * b[i] over 8 BF16 pairs, in element order, fused multiply-add.
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w};
  const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf(bf16_to_f32(av[i] & 0xffffu), bf16_to_f32(bv[i] & 0xffffu), acc);
    acc = __builtin_fmaf(bf16_to_f32(av[i] >> 16), bf16_to_f32(bv[i] >> 16), acc);
  }
  return acc;
}

__global__ __launch_bounds__(256) void gather_shrink_kernel(
    const uint16_t* __restrict__ x, uint32_t xs, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ row_adapter, uint32_t top_k, const uint64_t* __restrict__ a_table,
    const uint64_t* __restrict__ b_table, uint32_t max_loras, uint32_t E, uint32_t k_in,
    uint32_t R, uint16_t* __restrict__ xa) {
  const uint32_t rho = blockIdx.x;
  uint16_t* xo = xa + (size_t)rho * R;
  const int pair = gather_pair(rho, indices, row_adapter, top_k, a_table, b_table, max_loras, E);
  if (pair < 0) {
    for (uint32_t k = threadIdx.x; k < R; k += 256) xo[k] = 0;
    return;
  }
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a_table[pair]);
  const uint16_t* xr = x + (size_t)rho * xs;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (uint32_t k = wave; k < R; k += 4) {
    const uint16_t* Ak = A + (size_t)k * k_in;
    float acc = 0.f;
    for (uint32_t c = lane * 8; c < k_in; c += 512) acc = dot8(load16(xr + c), load16(Ak + c), acc);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) xo[k] = (uint16_t)f32_to_bf16(acc);
  }
}

__global__ __launch_bounds__(256) void gather_expand_kernel(
    const uint16_t* __restrict__ xa, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ row_adapter, uint32_t top_k, const uint64_t* __restrict__ a_table,
    const uint64_t* __restrict__ b_table, const float* __restrict__ scale_table,
    uint32_t max_loras, uint32_t E, uint32_t n_out, uint32_t R, uint16_t* __restrict__ out,
    uint32_t os) {
  const uint32_t rho = blockIdx.x;
  const int pair = gather_pair(rho, indices, row_adapter, top_k, a_table, b_table, max_loras, E);
  if (pair < 0) return;
  const uint32_t j = blockIdx.y * kGatherCols + threadIdx.x * 2;
  if (j >= n_out) return;
  const uint16_t* B0 = reinterpret_cast<const uint16_t*>(b_table[pair]) + (size_t)j * R;
  const uint16_t* B1 = B0 + R;
  const uint16_t* xr = xa + (size_t)rho * R;
  float d0 = 0.f, d1 = 0.f;
  for (uint32_t k = 0; k < R; k += 8) {
    const uint4 xv = load16(xr + k);
    d0 = dot8(load16(B0 + k), xv, d0);
    d1 = dot8(load16(B1 + k), xv, d1);
  }
  uint32_t* p = reinterpret_cast<uint32_t*>(out + (size_t)rho * os + j);
  const uint32_t dd = f32_to_bf16(d0) | (f32_to_bf16(d1) << 16);
  *p = fold2(*p, dd, scale_table[pair]);
}

// ----------------------------------------------------------------- grouped --

struct GroupedRows {
  const int32_t* off;
  const int32_t* stid;
  const int32_t* radapt;
  const uint64_t* a_table;
  const uint64_t* b_table;
  uint32_t E_off;
  uint32_t num_tokens;
  uint32_t max_loras;
  uint32_t E;
  int need_tok;
};

// (slot, expert) pair index of sorted row r, or -1 for a row that does not fold.
__device__ __forceinline__ int grouped_row_key(uint32_t r, const GroupedRows& g, int* tok) {
  const int e = expert_of_row(g.off, (int)g.E_off, (int)r);
  if (e < 0 || (uint32_t)e >= g.E) return -1;
  int t = 0;
  if (g.need_tok) {
    t = g.stid[r];
    if (t < 0 || (uint32_t)t >= g.num_tokens) return -1;
  }
  const int s = g.radapt ? g.radapt[t] : 0;
  if (s < 0 || (uint32_t)s >= g.max_loras) return -1;
  const int pair = s * (int)g.E + e;
  if (g.a_table[pair] == 0ull || g.b_table[pair] == 0ull) return -1;
  *tok = t;
  return pair;
}

__global__ __launch_bounds__(256) void grouped_shrink_kernel(
    const uint16_t* __restrict__ x, uint32_t xs, int x_gather, GroupedRows gr, uint32_t k_in,
    uint32_t R, uint32_t row_offset, uint32_t row_end, uint32_t total, uint32_t ntr,
    uint16_t* __restrict__ xa) {
  __shared__ TileGroups tg;
  const uint32_t w = xcd_work_item(total);
  if (w >= total) return;
  const uint32_t rt = w % ntr;
  const uint32_t r0 = row_offset + (w / ntr) * RLD_M_TILE;
  if (r0 >= row_end) return;
  const int nr = (int)min((uint32_t)RLD_M_TILE, row_end - r0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (wave == 0) {
    int tok = 0;
    const int key = lane < nr ? grouped_row_key(r0 + lane, gr, &tok) : -1;
    group_tile_rows(key, tok, tg);
  }
  __syncthreads();

  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t col = rt * 16 + cl;
  const bool col_ok = col < R;
  // rows that do not fold get zero xa (this block's 16 columns)
  for (int e = threadIdx.x; e < nr * 16; e += 256) {
    const int l = e >> 4;
    const uint32_t cc = rt * 16 + (e & 15);
    if (tg.rowgrp[l] < 0 && cc < R) xa[(size_t)(r0 - row_offset + l) * R + cc] = 0;
  }

  // work units (group, 16-row subtile), spread over the waves
  const int ng = tg.ngroups;
  int unit = 0;
  for (int gi = 0; gi < ng; ++gi) {
    const int cnt = tg.gcount[gi];
    const int gs = tg.gstart[gi];
    const int nq = (cnt + 15) >> 4;
    for (int q = 0; q < nq; ++q, ++unit) {
      if ((unit & 3) != wave) continue;
      const uint16_t* A = reinterpret_cast<const uint16_t*>(gr.a_table[tg.gkey[gi]]);
      const uint16_t* Arow = A + (size_t)(col_ok ? col : 0) * k_in;
      const int li = q * 16 + cl;
      const bool ok = li < cnt;
      const int lrow = ok ? tg.grow[gs + li] : 0;
      const uint32_t xrow_idx = x_gather ? (uint32_t)tg.tok[lrow] : r0 + lrow;
      const uint16_t* xr = x + (size_t)xrow_idx * xs;
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
      for (uint32_t k0 = 0; k0 < k_in; k0 += 32) {
        const uint32_t k = k0 + lg * 8;
        const bool kok = k < k_in;
        const uint4 bop = (col_ok && kok) ? load16(Arow + k) : zero16();
        const uint4 aop = (ok && kok) ? load16(xr + k) : zero16();
        acc = mfma_bf16_16x16x32(aop, bop, acc);
      }
      if (col_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int l2 = q * 16 + 4 * lg + i;
          if (l2 < cnt) {
            const int lr = tg.grow[gs + l2];
            xa[(size_t)(r0 - row_offset + lr) * R + col] = (uint16_t)f32_to_bf16(acc[i]);
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void grouped_expand_kernel(
    const uint16_t* __restrict__ xa, GroupedRows gr, const float* __restrict__ scale_table,
    uint32_t n_out, uint32_t R, uint32_t row_offset, uint32_t row_end, uint32_t total,
    uint32_t nct, uint16_t* __restrict__ out, uint32_t os) {
  __shared__ TileGroups tg;
  __shared__ float srow[RLD_M_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t dl[RLD_M_TILE * kDlStride];
  const uint32_t w = xcd_work_item(total);
  if (w >= total) return;
  const uint32_t ct = w % nct;
  const uint32_t r0 = row_offset + (w / nct) * RLD_M_TILE;
  if (r0 >= row_end) return;
  const int nr = (int)min((uint32_t)RLD_M_TILE, row_end - r0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (wave == 0) {
    int tok = 0;
    const int key = lane < nr ? grouped_row_key(r0 + lane, gr, &tok) : -1;
    srow[lane] = key >= 0 ? scale_table[key] : 0.f;
    group_tile_rows(key, tok, tg);
  }
  __syncthreads();
  const int ng = tg.ngroups;
  if (ng == 0) return;

  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t j0 = ct * kJT;
  const int nks = (int)((R + 31) / 32);
  for (int gi = 0; gi < ng; ++gi) {
    const uint16_t* B = reinterpret_cast<const uint16_t*>(gr.b_table[tg.gkey[gi]]);
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
    const int cnt = tg.gcount[gi];
    const int gs = tg.gstart[gi];
    for (int p = 0; p * 16 < cnt; ++p) {
      const int li = p * 16 + cl;
      const bool ok = li < cnt;
      const int lrow = ok ? tg.grow[gs + li] : 0;
      const uint16_t* xr = xa + (size_t)(r0 - row_offset + lrow) * R;
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
        if (ok) {
          const uint32_t d01 = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
          const uint32_t d23 = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
          *reinterpret_cast<uint2*>(&dl[lrow * kDlStride + wave * 64 + m * 16 + 4 * lg]) =
              make_uint2(d01, d23);
        }
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nr * (kJT / 8); e += 256) {
    const int rl = e / (kJT / 8);
    const int c8 = (e % (kJT / 8)) * 8;
    const uint32_t col = j0 + c8;
    if (tg.rowgrp[rl] >= 0 && col < n_out) {
      uint16_t* p = out + (size_t)(r0 + rl) * os + col;
      const uint4 bv = *reinterpret_cast<const uint4*>(p);
      const uint4 dv = *reinterpret_cast<const uint4*>(&dl[rl * kDlStride + c8]);
      *reinterpret_cast<uint4*>(p) = fold8(bv, dv, srow[rl]);
    }
  }
}

}  // namespace rld

using namespace rld;

static int check_gather(const rld_moe_route* route, const int32_t* indices, uint32_t top_k,
                        uint32_t n_rows) {
  int st = check_moe_route(route);
  if (st) return st;
  if ((uint64_t)route->max_loras * route->num_experts > 0x7fffffffull) return RLD_EUNSUPPORTED;
  if (n_rows == 0) return RLD_OK;
  if (!indices || top_k == 0) return RLD_EINVAL;
  if (n_rows > 0x7fffffffu) return RLD_EUNSUPPORTED;
  return RLD_OK;
}

extern "C" int rld_moe_gather_shrink(const rld_moe_route* route, const void* x,
                                     uint32_t x_row_stride, const int32_t* indices,
                                     const int32_t* row_adapter, uint32_t top_k,
                                     uint32_t n_rows, void* xa, void* stream) {
  int st = check_gather(route, indices, top_k, n_rows);
  if (st || n_rows == 0) return st;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  hipLaunchKernelGGL(gather_shrink_kernel, dim3(n_rows), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                     x_row_stride, indices, row_adapter, top_k, route->a_table, route->b_table,
                     route->max_loras, route->num_experts, route->k_in, route->max_rank,
                     static_cast<uint16_t*>(xa));
  return launch_status();
}

extern "C" int rld_moe_gather_expand_fold(const rld_moe_route* route, const void* xa,
                                          const int32_t* indices, const int32_t* row_adapter,
                                          uint32_t top_k, uint32_t n_rows, void* base_out,
                                          uint32_t out_row_stride, void* stream) {
  int st = check_gather(route, indices, top_k, n_rows);
  if (st || n_rows == 0) return st;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  hipLaunchKernelGGL(gather_expand_kernel, dim3(n_rows, div_ceil(route->n_out, kGatherCols)),
                     dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(xa), indices, row_adapter, top_k,
                     route->a_table, route->b_table, route->scale_table, route->max_loras,
                     route->num_experts, route->n_out, route->max_rank,
                     static_cast<uint16_t*>(base_out), out_row_stride);
  return launch_status();
}

extern "C" int rld_moe_gather(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                              const int32_t* indices, const int32_t* row_adapter, uint32_t top_k,
                              uint32_t n_rows, void* base_out, uint32_t out_row_stride, void* xa,
                              void* stream) {
  int st = check_gather(route, indices, top_k, n_rows);
  if (st || n_rows == 0) return st;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  st = rld_moe_gather_shrink(route, x, x_row_stride, indices, row_adapter, top_k, n_rows, xa,
                             stream);
  if (st) return st;
  return rld_moe_gather_expand_fold(route, xa, indices, row_adapter, top_k, n_rows, base_out,
                                    out_row_stride, stream);
}

static int check_grouped(const rld_moe_route* route, int x_gather, const int32_t* expert_offsets,
                         uint32_t num_experts_off, const int32_t* sorted_token_ids,
                         const int32_t* row_adapter, uint32_t row_offset, uint32_t row_end) {
  int st = check_moe_route(route);
  if (st) return st;
  if ((uint64_t)route->max_loras * route->num_experts > 0x7fffffffull) return RLD_EUNSUPPORTED;
  if (!expert_offsets || num_experts_off == 0) return RLD_EINVAL;
  if (row_end < row_offset || row_end > 0x7fffffffu) return RLD_EINVAL;
  if ((x_gather || row_adapter) && !sorted_token_ids) return RLD_EINVAL;
  return RLD_OK;
}

static GroupedRows make_rows(const rld_moe_route* route, int x_gather, uint32_t num_tokens,
                             const int32_t* expert_offsets, uint32_t num_experts_off,
                             const int32_t* sorted_token_ids, const int32_t* row_adapter) {
  GroupedRows g;
  g.off = expert_offsets;
  g.stid = sorted_token_ids;
  g.radapt = row_adapter;
  g.a_table = route->a_table;
  g.b_table = route->b_table;
  g.E_off = num_experts_off;
  g.num_tokens = num_tokens;
  g.max_loras = route->max_loras;
  g.E = route->num_experts;
  g.need_tok = (x_gather || row_adapter) ? 1 : 0;
  return g;
}

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
  const uint32_t wc = rld_grouped_wc(row_offset, row_end);
  const uint32_t ntr = div_ceil(route->max_rank, 16);
  const uint32_t total = wc * ntr;
  GroupedRows gr = make_rows(route, x_gather, num_tokens, expert_offsets, num_experts_off,
                             sorted_token_ids, row_adapter);
  hipLaunchKernelGGL(grouped_shrink_kernel, dim3(xcd_grid(total)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                     x_row_stride, x_gather ? 1 : 0, gr, route->k_in, route->max_rank,
                     row_offset, row_end, total, ntr, static_cast<uint16_t*>(xa));
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
  const uint32_t wc = rld_grouped_wc(row_offset, row_end);
  const uint32_t nct = div_ceil(route->n_out, kJT);
  const uint32_t total = wc * nct;
  GroupedRows gr = make_rows(route, 0, num_tokens, expert_offsets, num_experts_off,
                             sorted_token_ids, row_adapter);
  hipLaunchKernelGGL(grouped_expand_kernel, dim3(xcd_grid(total)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint16_t*>(xa), gr,
                     route->scale_table, route->n_out, route->max_rank, row_offset, row_end,
                     total, nct, static_cast<uint16_t*>(base_out), out_row_stride);
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
