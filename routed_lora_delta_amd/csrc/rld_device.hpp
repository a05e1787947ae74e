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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round binary32 values to bfloat16, ties to even, with gfx950's
// v_cvt_pk_bf16_f32 (two values per instruction): round to nearest even on the
// 16 dropped significand bits, NaN -> quiet NaN with the sign kept, overflow ->
// infinity, subnormals rounded like normals.  (The instruction's results were
// checked against that definition on every exponent with tie, above-tie and
// below-tie patterns, on subnormals and around the largest finite value.)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ floatx4 mfma_bf16_16x16x32(const uint4& a, const uint4& b,
                                                      const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Device memory is reached only through address-space-1 (global) pointers,
// so every access compiles to global_load / global_store, which count on
// vmcnt alone.  A flat access (what a generic pointer gives) also counts on
// lgkmcnt, so every LDS wait and every barrier would wait for it as well and
// loads issued early could no longer overlap the work after them.  Addresses
// travel in kernel argument structs as uint64_t and become global pointers
// through gp().
#define RLD_GLOBAL __attribute__((address_space(1)))

template <class T>
__device__ __forceinline__ RLD_GLOBAL T* gp(uint64_t addr) {
  return (RLD_GLOBAL T*)addr;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const RLD_GLOBAL uint16_t* p) {
  const u32x4 v = *reinterpret_cast<const RLD_GLOBAL u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store16(RLD_GLOBAL uint16_t* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  *reinterpret_cast<RLD_GLOBAL u32x4*>(p) = w;
}

__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

// Compiler-level memory barrier: the loads written before it are issued
// before it (no load can be moved across it), without waiting for their data.
__device__ __forceinline__ void issue_point() { asm volatile("" ::: "memory"); }

// out = bf16(f32(base) + f32(scale * f32(delta))): the product is rounded to
// fp32 before the add (base += scale * bf16(delta) in fp32), never fused.
__device__ __forceinline__ float fold_f32(uint32_t base16, uint32_t delta16, float scale) {
#pragma clang fp contract(off)
  const float t = scale * bf16_to_f32(delta16);
  return bf16_to_f32(base16) + t;
}

__device__ __forceinline__ uint32_t fold2(uint32_t base2, uint32_t delta2, float scale) {
  return pack_bf16x2(fold_f32(base2 & 0xffffu, delta2 & 0xffffu, scale),
                     fold_f32(base2 >> 16, delta2 >> 16, scale));
}

__device__ __forceinline__ uint4 fold8(const uint4& base, const uint4& delta, float scale) {
  return make_uint4(fold2(base.x, delta.x, scale), fold2(base.y, delta.y, scale),
                    fold2(base.z, delta.z, scale), fold2(base.w, delta.w, scale));
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// A block of NW waves appends to `list` (LDS), in thread order, the `row` of
// every thread whose `hit` is set.  Returns the number appended (in every
// thread).  `wcount` is LDS scratch of NW ints.
template <int NW = 4>
__device__ __forceinline__ int append_hits(bool hit, uint32_t row, int* list, int base,
                                           int* wcount) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(hit);
  if (lane == 0) wcount[wave] = __popcll(m);
  __syncthreads();
  int off = base;
  int tot = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    off += (v < wave) ? wcount[v] : 0;
    tot += wcount[v];
  }
  if (hit) list[off + __popcll(m & lanemask_lt(lane))] = (int)row;
  __syncthreads();
  return tot;
}

// A block of 256 threads appends to `list` (LDS) the indices of rows in
// [pos, min(pos+256, n)) whose key equals `want`, in ascending order.
// Returns the number appended.  `wcount` is LDS scratch of 4 ints.
__device__ __forceinline__ int append_matching_rows(const RLD_GLOBAL int32_t* keys, uint32_t n,
                                                    uint32_t pos, int32_t want, int* list,
                                                    int base, int* wcount) {
  const uint32_t row = pos + threadIdx.x;
  return append_hits(row < n && keys[row] == want, row, list, base, wcount);
}

// Owner expert of sorted row r: the largest e < E with off[e] <= r, accepted
// only if r < off[e+1].  Reads stay inside off[0..E]; non-monotone offsets give
// some defined answer without faulting.  P is an LDS or a global pointer.
template <class P>
__device__ __forceinline__ int expert_of_row(P off, int E, int r) {
  if (E <= 0 || r < off[0]) return -1;
  int lo = 0, hi = E - 1;  // invariant: off[lo] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return r < off[lo + 1] ? lo : -1;
}

// Block-wide arrival on a counter shared by the blocks that each produce part
// of a result: this thread's stores have completed (the partial results were
// written with agent-scope stores, which other XCDs see), then the block
// meets, then thread 0 adds 1 to *ctr (agent scope) and every thread gets the
// old value in *slot (LDS).  The block that sees (arrivals - 1) is the last.
__device__ __forceinline__ uint32_t block_signal(RLD_GLOBAL uint32_t* ctr, int* slot) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *slot = (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t old = (uint32_t)*slot;
  __syncthreads();
  return old;
}

// Block index remap so that consecutive work items land on the same XCD
// (workgroups are dispatched round-robin over the 8 XCDs).  gridDim.x must be
// a multiple of 8; returns >= total for padding blocks.
__device__ __forceinline__ uint32_t xcd_work_item(uint32_t total) {
  const uint32_t per = gridDim.x >> 3;
  return (blockIdx.x & 7u) * per + (blockIdx.x >> 3);
}

// Block index remap that keeps each group of `group` consecutive work items on
// one XCD (they share inputs through that XCD's L2) and deals the groups out
// to the 8 XCDs in turn (so a run of heavy groups spreads over the chip).
// The grid must be 8 * group * ceil(ceil(total / group) / 8) blocks (see
// xcd_group_grid); returns >= total for padding blocks.
__device__ __forceinline__ uint32_t xcd_group_item(uint32_t group) {
  const uint32_t p = blockIdx.x >> 3;
  return ((p / group) * 8u + (blockIdx.x & 7u)) * group + p % group;
}

}  // namespace rld
