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
//   fold    rld_moe_gather: one block per row does both, the same arithmetic in
//           the same order (so the same bits), with the xa row passed through
//           LDS; the expand's launch, its routing loads and the xa read-back
//           are saved.
//
#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

// Kernel arguments of the gather fold; device addresses are integers read
// through global-pointer accessors (see gp()).
struct GatherArgs {
  uint64_t x_, idx_, radapt_, atab_, btab_, stab_, xa_, out_;
  uint32_t xs, top_k, max_loras, E, k_in, n_out, R, os;
  __device__ const RLD_GLOBAL uint16_t* x() const { return gp<const uint16_t>(x_); }
  __device__ const RLD_GLOBAL int32_t* indices() const { return gp<const int32_t>(idx_); }
  __device__ const RLD_GLOBAL int32_t* row_adapter() const { return gp<const int32_t>(radapt_); }
  __device__ const RLD_GLOBAL uint64_t* a_table() const { return gp<const uint64_t>(atab_); }
  __device__ const RLD_GLOBAL uint64_t* b_table() const { return gp<const uint64_t>(btab_); }
  __device__ const RLD_GLOBAL float* scale_table() const { return gp<const float>(stab_); }
  __device__ RLD_GLOBAL uint16_t* xa() const { return gp<uint16_t>(xa_); }
  __device__ RLD_GLOBAL uint16_t* out() const { return gp<uint16_t>(out_); }
};

// ------------------------------------------------------------------ gather --

__device__ __forceinline__ int gather_pair(const GatherArgs& a, uint32_t rho) {
  const int s = a.radapt_ ? a.row_adapter()[rho / a.top_k] : 0;
  const int e = a.indices()[rho];
  if (s < 0 || (uint32_t)s >= a.max_loras || e < 0 || (uint32_t)e >= a.E) return -1;
  const int pair = s * (int)a.E + e;
  const uint64_t ta = a.a_table()[pair], tb = a.b_table()[pair];  // both in flight together
  if (ta == 0ull || tb == 0ull) return -1;
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

// xa row of flat row rho (valid pair): each wave owns every fourth column, its
// lanes split k_in in 16-byte pieces, and the lane sums meet in a fixed
// xor-butterfly.  The BF16 values go to xo and, when given, to xl (LDS).
__device__ __forceinline__ void gather_shrink_row(const GatherArgs& a, uint32_t rho, int pair,
                                                  RLD_GLOBAL uint16_t* xo, uint16_t* xl) {
  const uint32_t R = a.R, k_in = a.k_in;
  const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(a.a_table()[pair]);
  const RLD_GLOBAL uint16_t* xr = a.x() + (size_t)rho * a.xs;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // columns k = wave + 4i, up to kCols at a time: the x piece and the A pieces
  // of all of them go out together; each column still sums its pieces in
  // ascending order
  constexpr int kCols = 8;
  for (uint32_t k0 = wave; k0 < R; k0 += 4 * kCols) {
    float acc[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i) acc[i] = 0.f;
    for (uint32_t c = lane * 8; c < k_in; c += 512) {
      const uint4 xv = load16(xr + c);
      uint4 av[kCols];
#pragma unroll
      for (int i = 0; i < kCols; ++i) {
        const uint32_t k = k0 + 4u * i;
        av[i] = load16(A + (size_t)(k < R ? k : k0) * k_in + c);
      }
#pragma unroll
      for (int i = 0; i < kCols; ++i) acc[i] = dot8(xv, av[i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < kCols; ++i) {
      const uint32_t k = k0 + 4u * i;
      float v = acc[i];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && k < R) {
        const uint16_t b = (uint16_t)f32_to_bf16(v);
        xo[k] = b;
        if (xl) xl[k] = b;
      }
    }
  }
}

// 8 xa values from global memory or from LDS.
__device__ __forceinline__ uint4 xa8(const RLD_GLOBAL uint16_t* p) { return load16(p); }
__device__ __forceinline__ uint4 xa8(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Output columns j, j + 1 of flat row rho: the sum over max_rank in order
// (xa from xr: global memory or LDS), folded into 4 bytes of base_out.
template <typename XP>
__device__ __forceinline__ void gather_fold_cols(const GatherArgs& a, uint32_t rho, int pair,
                                                 uint32_t j, XP xr) {
  const uint32_t R = a.R;
  const RLD_GLOBAL uint16_t* B0 = gp<const uint16_t>(a.b_table()[pair]) + (size_t)j * R;
  const RLD_GLOBAL uint16_t* B1 = B0 + R;
  float d0 = 0.f, d1 = 0.f;
  for (uint32_t k = 0; k < R; k += 8) {
    const uint4 xv = xa8(xr + k);
    d0 = dot8(load16(B0 + k), xv, d0);
    d1 = dot8(load16(B1 + k), xv, d1);
  }
  RLD_GLOBAL uint32_t* p = reinterpret_cast<RLD_GLOBAL uint32_t*>(a.out() + (size_t)rho * a.os + j);
  const uint32_t dd = pack_bf16x2(d0, d1);
  *p = fold2(*p, dd, a.scale_table()[pair]);
}

// Output columns [j, j + 8) of flat row rho, max_rank <= 16: the same sums
// and folds as gather_fold_cols, with the B rows of the eight columns, the base
// values and xa (LDS) in one round.
__device__ __forceinline__ void gather_fold_cols8(const GatherArgs& a, uint32_t rho, int pair,
                                                  uint32_t j, const uint16_t* xl) {
  const uint32_t R = a.R;
  const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(a.b_table()[pair]) + (size_t)j * R;
  RLD_GLOBAL uint16_t* op = a.out() + (size_t)rho * a.os + j;
  uint4 bv[8][2];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 2; ++q) bv[c][q] = load16(B + (size_t)c * R + (8u * q < R ? 8u * q : 0));
  const uint4 base = load16(op);
  float d[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    d[c] = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (8u * q < R) d[c] = dot8(bv[c][q], xa8(xl + 8 * q), d[c]);
  }
  const float scale = a.scale_table()[pair];
  const uint4 o = make_uint4(fold2(base.x, pack_bf16x2(d[0], d[1]), scale),
                             fold2(base.y, pack_bf16x2(d[2], d[3]), scale),
                             fold2(base.z, pack_bf16x2(d[4], d[5]), scale),
                             fold2(base.w, pack_bf16x2(d[6], d[7]), scale));
  store16(op, o);
}

__global__ __launch_bounds__(256) void gather_shrink_kernel(GatherArgs a) {
  const uint32_t rho = blockIdx.x;
  RLD_GLOBAL uint16_t* xo = a.xa() + (size_t)rho * a.R;
  const int pair = gather_pair(a, rho);
  if (pair < 0) {
    for (uint32_t k = threadIdx.x; k < a.R; k += 256) xo[k] = 0;
    return;
  }
  gather_shrink_row(a, rho, pair, xo, nullptr);
}

__global__ __launch_bounds__(256) void gather_expand_kernel(GatherArgs a) {
  const uint32_t rho = blockIdx.x;
  const int pair = gather_pair(a, rho);
  if (pair < 0) return;
  const uint32_t j = blockIdx.y * kGatherCols + threadIdx.x * 2;
  if (j >= a.n_out) return;
  gather_fold_cols(a, rho, pair, j, a.xa() + (size_t)rho * a.R);
}

// Shrink and fold of one flat row per block (rld_moe_gather): the two kernels
// above in one, the xa row handed over in LDS.
// Fold of flat row rho when max_rank <= 16, k_in <= 1024 and n_out <= 2048
// (one 8-column piece per thread): the row's loads go out in three rounds --
// its routing entries with its x and base values, the pair's table entries,
// then A_{s,e} and B_{s,e} together -- instead of one round per step.  The
// arithmetic is gather_shrink_row's and gather_fold_cols8's, in the same
// order (a lane's k pieces lane*8 + 512m in ascending m, the same
// xor-butterfly, the same rank order of the fold), so the bits are the same.
__device__ __forceinline__ void gather_fold_row_small(const GatherArgs& a, uint32_t rho,
                                                      uint16_t* xl) {
  const uint32_t R = a.R, k_in = a.k_in;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t j = threadIdx.x * 8u;
  const bool fold_j = j < a.n_out;
  RLD_GLOBAL uint16_t* op = a.out() + (size_t)rho * a.os + (fold_j ? j : 0u);
  const RLD_GLOBAL uint16_t* xr = a.x() + (size_t)rho * a.xs;
  // round 1: routing, x pieces, base values (clamped in-bounds addresses)
  const int s = a.radapt_ ? a.row_adapter()[rho / a.top_k] : 0;
  const int e = a.indices()[rho];
  uint4 xv[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t c = (uint32_t)lane * 8u + 512u * m;
    xv[m] = load16(xr + (c < k_in ? c : 0u));
  }
  const uint4 base = load16(op);
  issue_point();
  // round 2: the pair's table entries (index 0 when the routing is out of range)
  const bool in_range = s >= 0 && (uint32_t)s < a.max_loras && e >= 0 && (uint32_t)e < a.E;
  const int pair = in_range ? s * (int)a.E + e : 0;
  const uint64_t ta = a.a_table()[pair], tb = a.b_table()[pair];
  const float scale = a.scale_table()[pair];
  RLD_GLOBAL uint16_t* xo = a.xa() + (size_t)rho * R;
  if (!in_range || ta == 0ull || tb == 0ull) {
    for (uint32_t k = threadIdx.x; k < R; k += 256) xo[k] = 0;
    return;
  }
  // round 3: this wave's A_{s,e} rows k = wave + 4i and the B_{s,e} rows of
  // this thread's eight output columns
  const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(ta);
  const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(tb) + (fold_j ? (size_t)j * R : 0);
  uint4 av[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t k = (uint32_t)wave + 4u * i;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t c = (uint32_t)lane * 8u + 512u * m;
      av[i][m] = load16(A + (size_t)(k < R ? k : 0u) * k_in + (c < k_in ? c : 0u));
    }
  }
  uint4 bv[8][2];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      bv[c][q] = load16(B + (fold_j ? (size_t)c * R + (8u * q < R ? 8u * q : 0u) : 0u));
  issue_point();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t k = (uint32_t)wave + 4u * i;
    float v = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      if ((uint32_t)lane * 8u + 512u * m < k_in) v = dot8(xv[m], av[i][m], v);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && k < R) {
      const uint16_t b = (uint16_t)f32_to_bf16(v);
      xo[k] = b;
      xl[k] = b;
    }
  }
  __syncthreads();
  if (!fold_j) return;
  float d[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    d[c] = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (8u * q < R) d[c] = dot8(bv[c][q], xa8(xl + 8 * q), d[c]);
  }
  const uint4 o = make_uint4(fold2(base.x, pack_bf16x2(d[0], d[1]), scale),
                             fold2(base.y, pack_bf16x2(d[2], d[3]), scale),
                             fold2(base.z, pack_bf16x2(d[4], d[5]), scale),
                             fold2(base.w, pack_bf16x2(d[6], d[7]), scale));
  store16(op, o);
}

__global__ __launch_bounds__(256) void gather_fold_kernel(GatherArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xl[RLD_MAX_RANK];
  const uint32_t rho = blockIdx.x;
  if (a.R <= 16u && a.k_in <= 1024u && a.n_out <= 2048u) {
    gather_fold_row_small(a, rho, xl);
    return;
  }
  RLD_GLOBAL uint16_t* xo = a.xa() + (size_t)rho * a.R;
  const int pair = gather_pair(a, rho);
  if (pair < 0) {
    for (uint32_t k = threadIdx.x; k < a.R; k += 256) xo[k] = 0;
    return;
  }
  gather_shrink_row(a, rho, pair, xo, xl);
  __syncthreads();
  if (a.R <= 16) {
    // n_out is a multiple of 8
    for (uint32_t j = threadIdx.x * 8; j < a.n_out; j += 8 * 256)
      gather_fold_cols8(a, rho, pair, j, xl);
  } else {
    for (uint32_t j = threadIdx.x * 2; j < a.n_out; j += 2 * 256)
      gather_fold_cols(a, rho, pair, j, static_cast<const uint16_t*>(xl));
  }
}

static GatherArgs gather_args(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                              const int32_t* indices, const int32_t* row_adapter, uint32_t top_k,
                              const void* xa, void* base_out, uint32_t out_row_stride) {
  GatherArgs a = {};
  a.x_ = reinterpret_cast<uint64_t>(x);
  a.idx_ = reinterpret_cast<uint64_t>(indices);
  a.radapt_ = reinterpret_cast<uint64_t>(row_adapter);
  a.atab_ = reinterpret_cast<uint64_t>(route->a_table);
  a.btab_ = reinterpret_cast<uint64_t>(route->b_table);
  a.stab_ = reinterpret_cast<uint64_t>(route->scale_table);
  a.xa_ = reinterpret_cast<uint64_t>(xa);
  a.out_ = reinterpret_cast<uint64_t>(base_out);
  a.xs = x_row_stride;
  a.top_k = top_k;
  a.max_loras = route->max_loras;
  a.E = route->num_experts;
  a.k_in = route->k_in;
  a.n_out = route->n_out;
  a.R = route->max_rank;
  a.os = out_row_stride;
  return a;
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
                     reinterpret_cast<hipStream_t>(stream),
                     gather_args(route, x, x_row_stride, indices, row_adapter, top_k, xa,
                                 nullptr, 0));
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
                     gather_args(route, nullptr, 0, indices, row_adapter, top_k, xa, base_out,
                                 out_row_stride));
  return launch_status();
}

extern "C" int rld_moe_gather(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                              const int32_t* indices, const int32_t* row_adapter, uint32_t top_k,
                              uint32_t n_rows, void* base_out, uint32_t out_row_stride, void* xa,
                              void* stream) {
  int st = check_gather(route, indices, top_k, n_rows);
  if (st || n_rows == 0) return st;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  hipLaunchKernelGGL(gather_fold_kernel, dim3(n_rows), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     gather_args(route, x, x_row_stride, indices, row_adapter, top_k, xa,
                                 base_out, out_row_stride));
  return launch_status();
}
