// Host-side helpers shared by the launchers: argument checks and launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rld.h"

namespace rld {

void record_hip_error(hipError_t e);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool mult8(uint64_t v) { return (v & 7u) == 0; }
// ceil(a / b) without the wrap of a + b - 1 near 2^32
inline uint32_t div_ceil(uint32_t a, uint32_t b) { return a / b + (a % b != 0u ? 1u : 0u); }

// Checks common to every route: dims non-zero, multiples of 8, rank bound.
inline int check_dims(uint32_t k_in, uint32_t n_out, uint32_t max_rank) {
  if (k_in == 0 || n_out == 0 || max_rank == 0) return RLD_EINVAL;
  if (max_rank > RLD_MAX_RANK) return RLD_EUNSUPPORTED;
  if (!mult8(k_in) || !mult8(n_out) || !mult8(max_rank)) return RLD_EALIGN;
  return RLD_OK;
}

inline int check_route(const rld_route* r) {
  if (!r || !r->a_table || !r->b_table || !r->scale_table || r->max_loras == 0) return RLD_EINVAL;
  return check_dims(r->k_in, r->n_out, r->max_rank);
}

inline int check_moe_route(const rld_moe_route* r) {
  if (!r || !r->a_table || !r->b_table || !r->scale_table || r->max_loras == 0 ||
      r->num_experts == 0)
    return RLD_EINVAL;
  return check_dims(r->k_in, r->n_out, r->max_rank);
}

inline int check_rows(const void* p, uint32_t stride, uint32_t width) {
  if (!p) return RLD_EINVAL;
  if (stride < width) return RLD_EINVAL;
  if (!mult8(stride) || !aligned16(p)) return RLD_EALIGN;
  return RLD_OK;
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    record_hip_error(e);
    return RLD_ELAUNCH;
  }
  return RLD_OK;
}

// k_in split of the BGMV shrink: a function of (k_in, max_rank) only, so a row's
// summation order never depends on the batch.  Narrow ranks get shorter chunks
// so that a call still spreads over many blocks.
inline uint32_t bgmv_chunk(uint32_t k_in, uint32_t max_rank) {
  const uint32_t kc = max_rank <= 16 ? 256u : 512u;
  return k_in <= kc ? k_in : kc;
}

// Waves of a BGMV shrink block: the chunk's 32-wide K steps are dealt to them
// round robin, and their sums are added in wave order, so this is part of the
// summation order and a function of (k_in, max_rank) only.  Eight waves of two
// steps hold the x fragments of 128 rows in the registers four waves of four
// steps need for 64, so a slot with up to 128 rows of the batch is one round of
// loads.
inline uint32_t bgmv_shrink_waves(uint32_t k_in, uint32_t max_rank) {
  (void)k_in;
  return max_rank > 16 ? 8u : 4u;
}

// 16-column MFMA tiles of xa per BGMV shrink item.  Routed calls take 1 or 2
// (wider ranks take several column groups: four tiles' operands leave the
// kernel two waves per SIMD, two tiles three).  The unrouted mode takes up to
// 4: each of its items reads a whole 64-row x tile, which every further
// column group would read again.
inline uint32_t bgmv_nt(uint32_t max_rank, bool unrouted = false) {
  const uint32_t t = div_ceil(max_rank, 16u);
  return t <= 1u ? 1u : (t <= 2u || !unrouted ? 2u : 4u);
}

// Grid of xcd_group_item: 8 XCDs x whole groups, covering `total` items.
inline uint32_t xcd_group_grid(uint32_t total, uint32_t group) {
  return 8u * group * div_ceil(div_ceil(total, group), 8u);
}

// Wide MoE grouped shrink: for 1024 < k_in <= 2048 and max_rank <= 32 one
// block of 16 waves covers the whole of k_in (128 k per wave), so no partials
// and no second pass are needed.
inline bool grouped_wide(uint32_t k_in, uint32_t max_rank) {
  return k_in > 1024u && k_in <= 2048u && max_rank <= 32u;
}

// k chunk of the MoE grouped shrink, a function of (k_in, max_rank) only (so a
// row's summation order never depends on its window): up to k_in = 1024 the
// whole of k_in in one chunk of 512, 768 or 1024 (four waves, no partials, no
// reduce); the wide case above in one chunk of 2048 (sixteen waves); otherwise
// chunks of 512 (four waves x 128 k).
inline uint32_t grouped_chunk(uint32_t k_in, uint32_t max_rank) {
  if (grouped_wide(k_in, max_rank)) return 2048u;
  if (k_in > 1024u) return 512u;
  return k_in <= 512u ? 512u : (k_in <= 768u ? 768u : 1024u);
}

// 16-column MFMA tiles of xa held by one grouped shrink item (1, 2 or 4).
inline uint32_t grouped_nt(uint32_t max_rank) {
  const uint32_t t = div_ceil(max_rank, 16u);
  return t <= 1u ? 1u : (t <= 2u ? 2u : 4u);
}

// Workspace of a grouped shrink window of `rows` rows: fp32 partials
// [chunks][rows][max_rank] (16-byte rounded) plus 16 bytes of counter per
// (slot, expert) pair; none when k_in fits one chunk.
inline size_t grouped_workspace(uint32_t rows, uint32_t k_in, uint32_t max_rank,
                                uint32_t max_loras, uint32_t num_experts) {
  if (k_in == 0 || max_rank == 0 || max_loras == 0 || num_experts == 0) return 0;
  const uint32_t nch = div_ceil(k_in, grouped_chunk(k_in, max_rank));
  if (nch == 1) return 0;
  const size_t part = ((size_t)nch * rows * max_rank * 4 + 15) & ~(size_t)15;
  return part + (size_t)16 * max_loras * num_experts;
}

// Blocks of the persistent grouped shrink launch (fewer when there are fewer
// possible items): 256-thread blocks, or 1024-thread blocks of the wide case.
constexpr uint32_t kGsGrid = 512;
constexpr uint32_t kGwGrid = 256;

// Output columns per block of the gather expand (two per thread).
constexpr uint32_t kGatherCols = 512;

// Grid padded to a multiple of 8 for the XCD remap.
inline uint32_t xcd_grid(uint32_t total) { return 8u * div_ceil(total, 8u); }

}  // namespace rld
