// MoE decode gather-fold ("Module moe_lora_grouped", moe_lora_gather_bgmv).
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
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

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
  const uint32_t dd = pack_bf16x2(d0, d1);
  *p = fold2(*p, dd, scale_table[pair]);
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
