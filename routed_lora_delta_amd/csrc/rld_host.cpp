// Host-only parts of the C ABI: install-time table packing, the pure launch
// helpers of "Module moe_lora_grouped", and diagnostics.  Nothing here touches
// a device.
#include <math.h>
#include <string.h>

#include "rld_internal.hpp"

namespace rld {

static thread_local int g_last_hip_error = 0;

void record_hip_error(hipError_t e) { g_last_hip_error = static_cast<int>(e); }

static int check_entry(const rld_adapter_entry& e, uint32_t max_loras, uint32_t max_rank) {
  if (e.slot >= max_loras || e.rank == 0 || e.rank > max_rank) return RLD_EINVAL;
  if (e.a_addr == 0 || e.b_addr == 0) return RLD_EINVAL;
  if ((e.a_addr & 15u) || (e.b_addr & 15u)) return RLD_EALIGN;
  return RLD_OK;
}

}  // namespace rld

using namespace rld;

extern "C" int rld_scale(float alpha, uint32_t rank, int use_rslora, float* out) {
  if (!out || rank == 0) return RLD_EINVAL;
  const double a = static_cast<double>(alpha);
  const double r = static_cast<double>(rank);
  *out = static_cast<float>(use_rslora ? a / sqrt(r) : a / r);
  return RLD_OK;
}

// F16 -> F32, exact: F32 has more exponent and significand bits than F16,
// and F16 subnormals are F32 normals.
static uint32_t f16_bits_to_f32_bits(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu;
  uint32_t m = h & 0x3ffu;
  if (e == 0x1fu) return sign | 0x7f800000u | (m << 13);  // Inf, NaN (payload kept)
  if (e != 0) return sign | ((e + 112u) << 23) | (m << 13);
  if (m == 0) return sign;  // +-0
  // subnormal m * 2^-24: shift the leading one to bit 10
  int p = 0;
  while (!(m & 0x400u)) {
    m <<= 1;
    ++p;
  }
  return sign | ((uint32_t)(113 - p) << 23) | ((m & 0x3ffu) << 13);
}

// F32 bits -> BF16 bits, round to nearest on the 16 dropped bits, ties to
// even; NaN -> quiet NaN with the sign kept.
static uint16_t f32_bits_to_bf16(uint32_t u) {
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
    return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

extern "C" int rld_f16_to_bf16_host(const uint16_t* src, uint16_t* dst, size_t n) {
  if (n && (!src || !dst)) return RLD_EINVAL;
  for (size_t i = 0; i < n; ++i) dst[i] = f32_bits_to_bf16(f16_bits_to_f32_bits(src[i]));
  return RLD_OK;
}

extern "C" int rld_pad_adapter_host(const uint16_t* a, const uint16_t* b, uint32_t rank,
                                    uint32_t k_in, uint32_t n_out, uint32_t max_rank,
                                    uint16_t* a_pad, uint16_t* b_pad) {
  if (!a || !b || !a_pad || !b_pad || rank == 0 || rank > max_rank || k_in == 0 || n_out == 0)
    return RLD_EINVAL;
  memset(a_pad, 0, sizeof(uint16_t) * (size_t)max_rank * k_in);
  memcpy(a_pad, a, sizeof(uint16_t) * (size_t)rank * k_in);
  memset(b_pad, 0, sizeof(uint16_t) * (size_t)n_out * max_rank);
  for (uint32_t j = 0; j < n_out; ++j)
    memcpy(b_pad + (size_t)j * max_rank, b + (size_t)j * rank, sizeof(uint16_t) * rank);
  return RLD_OK;
}

extern "C" int rld_route_pack(const rld_adapter_entry* entries, size_t n_entries,
                              uint32_t max_loras, uint32_t max_rank, uint64_t* a_out,
                              uint64_t* b_out, float* scale_out) {
  if (!a_out || !b_out || !scale_out || max_loras == 0 || (n_entries && !entries))
    return RLD_EINVAL;
  for (size_t i = 0; i < n_entries; ++i) {
    const int st = check_entry(entries[i], max_loras, max_rank);
    if (st) return st;
  }
  for (uint32_t s = 0; s < max_loras; ++s) {
    a_out[s] = 0;
    b_out[s] = 0;
    scale_out[s] = 0.0f;
  }
  for (size_t i = 0; i < n_entries; ++i) {
    const rld_adapter_entry& e = entries[i];
    a_out[e.slot] = e.a_addr;
    b_out[e.slot] = e.b_addr;
    rld_scale(e.alpha, e.rank, e.use_rslora, &scale_out[e.slot]);
  }
  return RLD_OK;
}

extern "C" int rld_moe_tables_pack(const rld_adapter_entry* entries, size_t n_entries,
                                   uint32_t max_loras, uint32_t num_experts, uint32_t max_rank,
                                   uint64_t* a_out, uint64_t* b_out, float* scale_out) {
  if (!a_out || !b_out || !scale_out || max_loras == 0 || num_experts == 0 ||
      (n_entries && !entries))
    return RLD_EINVAL;
  for (size_t i = 0; i < n_entries; ++i) {
    const int st = check_entry(entries[i], max_loras, max_rank);
    if (st) return st;
    if (entries[i].expert < 0 || (uint32_t)entries[i].expert >= num_experts) return RLD_EINVAL;
  }
  const size_t tot = (size_t)max_loras * num_experts;
  for (size_t i = 0; i < tot; ++i) {
    a_out[i] = 0;
    b_out[i] = 0;
    scale_out[i] = 0.0f;
  }
  for (size_t i = 0; i < n_entries; ++i) {
    const rld_adapter_entry& e = entries[i];
    const size_t idx = (size_t)e.slot * num_experts + (uint32_t)e.expert;
    a_out[idx] = e.a_addr;
    b_out[idx] = e.b_addr;
    rld_scale(e.alpha, e.rank, e.use_rslora, &scale_out[idx]);
  }
  return RLD_OK;
}

extern "C" int rld_pack_expert_tables(const uint32_t* expert_ids, const uint64_t* a_addrs,
                                      const uint64_t* b_addrs, const float* scales,
                                      size_t n_entries, uint32_t cap, uint64_t* a_out,
                                      uint64_t* b_out, float* scale_out,
                                      uint32_t* n_experts_out) {
  if (!n_experts_out) return RLD_EINVAL;
  *n_experts_out = 0;
  if (n_entries == 0) return RLD_OK;
  if (!expert_ids || !a_addrs || !b_addrs || !scales || !a_out || !b_out || !scale_out)
    return RLD_EINVAL;
  uint64_t n = 0;
  for (size_t i = 0; i < n_entries; ++i)
    if ((uint64_t)expert_ids[i] + 1 > n) n = (uint64_t)expert_ids[i] + 1;
  if (n > cap) return RLD_ENOSPACE;
  for (uint64_t e = 0; e < n; ++e) {
    a_out[e] = 0;
    b_out[e] = 0;
    scale_out[e] = 0.0f;
  }
  for (size_t i = 0; i < n_entries; ++i) {
    a_out[expert_ids[i]] = a_addrs[i];
    b_out[expert_ids[i]] = b_addrs[i];
    scale_out[expert_ids[i]] = scales[i];
  }
  *n_experts_out = (uint32_t)n;
  return RLD_OK;
}

extern "C" int rld_grouped_windows(uint32_t total_rows, uint32_t cap, uint32_t* starts,
                                   uint32_t* ends, uint32_t max_windows, uint32_t* count) {
  if (!count || cap == 0) return RLD_EINVAL;
  const uint32_t n = total_rows == 0 ? 0 : div_ceil(total_rows, cap);
  *count = n;
  if (n > max_windows) return RLD_ENOSPACE;
  if (n && (!starts || !ends)) return RLD_EINVAL;
  for (uint32_t k = 0; k < n; ++k) {
    starts[k] = k * cap;
    const uint64_t e = (uint64_t)(k + 1) * cap;
    ends[k] = e < total_rows ? (uint32_t)e : total_rows;
  }
  return RLD_OK;
}

extern "C" uint32_t rld_grouped_wc(uint32_t row_offset, uint32_t row_end) {
  if (row_end < row_offset) return 0;
  const uint32_t len = row_end - row_offset;
  const uint32_t wc = len / RLD_M_TILE + (len % RLD_M_TILE ? 1u : 0u);
  return wc < 1 ? 1 : wc;
}

extern "C" uint32_t rld_gather_row_token(uint32_t row, uint32_t top_k) {
  return top_k == 0 ? 0 : row / top_k;
}

extern "C" int rld_gather_grids(uint32_t max_rank, uint32_t n_out, uint32_t n_rows,
                                uint32_t out[12]) {
  if (!out) return RLD_EINVAL;
  (void)max_rank;
  const uint32_t g[12] = {n_rows, 1, 1, 256, 1, 1, n_rows, div_ceil(n_out, kGatherCols), 1, 256, 1, 1};
  memcpy(out, g, sizeof(g));
  return RLD_OK;
}

extern "C" const char* rld_status_string(int status) {
  switch (status) {
    case RLD_OK: return "ok";
    case RLD_EINVAL: return "invalid argument";
    case RLD_EALIGN: return "misaligned size, stride, offset or pointer";
    case RLD_EUNSUPPORTED: return "unsupported size";
    case RLD_ELAUNCH: return "kernel launch failed";
    case RLD_ENOSPACE: return "scratch or output buffer too small";
    default: return "unknown status";
  }
}

extern "C" int rld_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char* rld_version(void) { return "rld 0.1 gfx950"; }
