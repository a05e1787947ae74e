// Device building blocks of the routed LoRA fold on gfx950 (CDNA4, wave64).
//
// BF16 values travel as their uint16 bit patterns.  Contractions run on the
// matrix cores through v_mfma_f32_16x16x32_bf16 (16x16 output tile, K = 32 per
// instruction, fp32 accumulate).  Operand layout used here, per lane l of the
// wave (g = l / 16, c = l % 16):
//   A operand  (16 x 32, M x K): row m = c, elements k = 8g .. 8g+7 (16 bytes)
//   B operand  (32 x 16, K x N): column n = c, elements k = 8g .. 8g+7
//   D          (16 x 16)       : D[4g + i][c] in element i of the float4
// A and B use the same (g, element) -> k assignment, so the product is the
// dot product over the 32 k values whatever order the hardware sums them in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rld {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round a binary32 value to bfloat16, ties to even (IEEE 754 roundTiesToEven
// applied to the 16 dropped significand bits).  NaN -> quiet NaN with the sign
// kept; overflow -> infinity; subnormals are rounded like normals (the bit
// pattern spacing is uniform across the subnormal/normal boundary).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x0040u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ floatx4 mfma_bf16_16x16x32(const uint4& a, const uint4& b,
                                                      const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

// out = bf16(f32(base) + f32(scale * f32(delta))): the product is rounded to
// fp32 before the add (base += scale * bf16(delta) in fp32), never fused.
__device__ __forceinline__ uint32_t fold1(uint32_t base16, uint32_t delta16, float scale) {
#pragma clang fp contract(off)
  const float t = scale * bf16_to_f32(delta16);
  const float s = bf16_to_f32(base16) + t;
  return f32_to_bf16(s);
}

__device__ __forceinline__ uint32_t fold2(uint32_t base2, uint32_t delta2, float scale) {
  const uint32_t lo = fold1(base2 & 0xffffu, delta2 & 0xffffu, scale);
  const uint32_t hi = fold1(base2 >> 16, delta2 >> 16, scale);
  return lo | (hi << 16);
}

__device__ __forceinline__ uint4 fold8(const uint4& base, const uint4& delta, float scale) {
  return make_uint4(fold2(base.x, delta.x, scale), fold2(base.y, delta.y, scale),
                    fold2(base.z, delta.z, scale), fold2(base.w, delta.w, scale));
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// A block of 256 threads appends to `list` (LDS) the indices of rows in
// [pos, min(pos+256, n)) whose key equals `want`, in ascending order.
// Returns the number appended.  `wcount` is LDS scratch of 4 ints.
__device__ __forceinline__ int append_matching_rows(const int32_t* __restrict__ keys, uint32_t n,
                                                    uint32_t pos, int32_t want, int* list,
                                                    int base, int* wcount) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t row = pos + threadIdx.x;
  const bool hit = row < n && keys[row] == want;
  const uint64_t m = __ballot(hit);
  if (lane == 0) wcount[wave] = __popcll(m);
  __syncthreads();
  int off = base;
  int tot = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    off += (v < wave) ? wcount[v] : 0;
    tot += wcount[v];
  }
  if (hit) list[off + __popcll(m & lanemask_lt(lane))] = (int)row;
  __syncthreads();
  return tot;
}

// Row classification of one grouped m-tile.  For tile rows r0 + l (l < nr),
// `key` is the (slot, expert) pair index s*E + e of a row that folds, or -1.
// Rows are grouped by key in first-occurrence order; within a group rows stay
// ascending.  Run by one full wave (lane = tile row); results in LDS.
struct TileGroups {
  int ngroups;
  int gkey[64];
  int gstart[64];
  int gcount[64];
  int grow[64];    // tile-local rows, grouped
  int rowgrp[64];  // group of each tile row, or -1
  int tok[64];     // token of each tile row (gather source)
};

__device__ __forceinline__ void group_tile_rows(int key, int tok, TileGroups& tg) {
  const int lane = threadIdx.x & 63;
  tg.rowgrp[lane] = -1;
  tg.tok[lane] = tok;
  uint64_t pending = __ballot(key >= 0);
  int ng = 0;
  int start = 0;
  while (pending) {
    const int leader = __ffsll((long long)pending) - 1;
    const int lk = __shfl(key, leader);
    const uint64_t m = __ballot(key == lk);
    const int cnt = __popcll(m);
    if (lane == 0) {
      tg.gkey[ng] = lk;
      tg.gstart[ng] = start;
      tg.gcount[ng] = cnt;
    }
    if (key == lk) {
      tg.grow[start + __popcll(m & lanemask_lt(lane))] = lane;
      tg.rowgrp[lane] = ng;
    }
    start += cnt;
    ++ng;
    pending &= ~m;
  }
  if (lane == 0) tg.ngroups = ng;
}

// Owner expert of sorted row r: the largest e < E with off[e] <= r, accepted
// only if r < off[e+1].  Reads stay inside off[0..E]; non-monotone offsets give
// some defined answer without faulting.
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ off, int E, int r) {
  if (E <= 0 || r < off[0]) return -1;
  int lo = 0, hi = E - 1;  // invariant: off[lo] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return r < off[lo + 1] ? lo : -1;
}

// Block index remap so that consecutive work items land on the same XCD
// (workgroups are dispatched round-robin over the 8 XCDs).  gridDim.x must be
// a multiple of 8; returns >= total for padding blocks.
__device__ __forceinline__ uint32_t xcd_work_item(uint32_t total) {
  const uint32_t per = gridDim.x >> 3;
  return (blockIdx.x & 7u) * per + (blockIdx.x >> 3);
}

}  // namespace rld
