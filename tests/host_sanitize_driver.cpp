// Host-only checks of librld's install and launch helpers, built together with
// routed_lora_delta_amd/csrc/rld_host.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py (no GPU involved).
// Every helper is called at its edges: exact-size buffers (heap allocations
// with nothing past their end, so any overrun is reported), empty inputs,
// repeated and out-of-range entries, and sizes near 2^32.  Exit status 0 and a
// last line "ok" when every result is the expected one.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "rld.h"

static int g_fail = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static rld_adapter_entry entry(uint32_t slot, int32_t expert, uint64_t a, uint64_t b,
                               uint32_t rank, float alpha, int rs) {
  rld_adapter_entry e;
  memset(&e, 0, sizeof(e));
  e.slot = slot;
  e.expert = expert;
  e.a_addr = a;
  e.b_addr = b;
  e.rank = rank;
  e.alpha = alpha;
  e.use_rslora = rs;
  return e;
}

static void check_scale() {
  float s = -1.f;
  EXPECT(rld_scale(16.f, 8, 0, &s) == RLD_OK && s == 2.0f);
  EXPECT(rld_scale(32.f, 64, 1, &s) == RLD_OK && s == 4.0f);
  EXPECT(rld_scale(16.f, 0, 0, &s) == RLD_EINVAL);
  EXPECT(rld_scale(16.f, 8, 0, nullptr) == RLD_EINVAL);
}

static void check_f16() {
  // all 65536 patterns through exact-size heap buffers
  std::vector<uint16_t> src(65536), dst(65536);
  for (uint32_t i = 0; i < 65536; ++i) src[i] = (uint16_t)i;
  EXPECT(rld_f16_to_bf16_host(src.data(), dst.data(), src.size()) == RLD_OK);
  EXPECT(dst[0x3c00] == 0x3f80);  // 1.0
  EXPECT(dst[0xbc00] == 0xbf80);  // -1.0
  EXPECT(dst[0x7c00] == 0x7f80);  // +inf
  EXPECT(dst[0x0001] == 0x3380);  // smallest subnormal, 2^-24
  EXPECT(rld_f16_to_bf16_host(nullptr, nullptr, 0) == RLD_OK);
  EXPECT(rld_f16_to_bf16_host(nullptr, dst.data(), 1) == RLD_EINVAL);
}

static void check_pad() {
  for (uint32_t rank : {1u, 5u, 8u}) {
    const uint32_t k_in = 24, n_out = 16, R = 8;
    uint16_t* a = (uint16_t*)malloc(sizeof(uint16_t) * rank * k_in);
    uint16_t* b = (uint16_t*)malloc(sizeof(uint16_t) * n_out * rank);
    uint16_t* ap = (uint16_t*)malloc(sizeof(uint16_t) * R * k_in);
    uint16_t* bp = (uint16_t*)malloc(sizeof(uint16_t) * n_out * R);
    for (uint32_t i = 0; i < rank * k_in; ++i) a[i] = (uint16_t)(i + 1);
    for (uint32_t i = 0; i < n_out * rank; ++i) b[i] = (uint16_t)(i + 7);
    EXPECT(rld_pad_adapter_host(a, b, rank, k_in, n_out, R, ap, bp) == RLD_OK);
    EXPECT(ap[(rank - 1) * k_in] == (uint16_t)((rank - 1) * k_in + 1));
    if (rank < R) EXPECT(ap[rank * k_in] == 0 && bp[rank] == 0);
    EXPECT(bp[(n_out - 1) * R + rank - 1] == (uint16_t)((n_out - 1) * rank + rank - 1 + 7));
    free(a);
    free(b);
    free(ap);
    free(bp);
  }
  uint16_t x[8] = {0};
  EXPECT(rld_pad_adapter_host(x, x, 9, 1, 1, 8, x, x) == RLD_EINVAL);  // rank > max_rank
  EXPECT(rld_pad_adapter_host(x, x, 0, 1, 1, 8, x, x) == RLD_EINVAL);
}

static void check_route_pack() {
  const uint32_t L = 4;
  uint64_t* a = (uint64_t*)malloc(sizeof(uint64_t) * L);
  uint64_t* b = (uint64_t*)malloc(sizeof(uint64_t) * L);
  float* s = (float*)malloc(sizeof(float) * L);
  rld_adapter_entry e[3] = {entry(3, -1, 0x1000, 0x2000, 8, 16.f, 0),
                            entry(0, -1, 0x3000, 0x4000, 4, 16.f, 0),
                            entry(3, -1, 0x5000, 0x6000, 16, 16.f, 1)};  // repeat: the last wins
  EXPECT(rld_route_pack(e, 3, L, 16, a, b, s) == RLD_OK);
  EXPECT(a[3] == 0x5000 && b[3] == 0x6000 && s[3] == 4.0f);
  EXPECT(a[0] == 0x3000 && s[0] == 4.0f);
  EXPECT(a[1] == 0 && b[2] == 0 && s[1] == 0.0f);
  rld_adapter_entry bad = entry(4, -1, 0x1000, 0x2000, 8, 16.f, 0);  // slot past the table
  EXPECT(rld_route_pack(&bad, 1, L, 16, a, b, s) == RLD_EINVAL);
  bad = entry(0, -1, 0x1008, 0x2000, 8, 16.f, 0);  // misaligned A
  EXPECT(rld_route_pack(&bad, 1, L, 16, a, b, s) == RLD_EALIGN);
  EXPECT(rld_route_pack(nullptr, 0, L, 16, a, b, s) == RLD_OK && a[3] == 0);
  free(a);
  free(b);
  free(s);
}

static void check_moe_pack() {
  const uint32_t L = 2, E = 5;
  uint64_t* a = (uint64_t*)malloc(sizeof(uint64_t) * L * E);
  uint64_t* b = (uint64_t*)malloc(sizeof(uint64_t) * L * E);
  float* s = (float*)malloc(sizeof(float) * L * E);
  rld_adapter_entry e[2] = {entry(1, 4, 0x1000, 0x2000, 8, 16.f, 0),
                            entry(0, 0, 0x3000, 0x4000, 8, 16.f, 0)};
  EXPECT(rld_moe_tables_pack(e, 2, L, E, 16, a, b, s) == RLD_OK);
  EXPECT(a[1 * E + 4] == 0x1000 && a[0] == 0x3000 && a[1] == 0 && s[9] == 2.0f);
  rld_adapter_entry bad = entry(0, 5, 0x1000, 0x2000, 8, 16.f, 0);  // expert past the table
  EXPECT(rld_moe_tables_pack(&bad, 1, L, E, 16, a, b, s) == RLD_EINVAL);
  bad = entry(0, -1, 0x1000, 0x2000, 8, 16.f, 0);
  EXPECT(rld_moe_tables_pack(&bad, 1, L, E, 16, a, b, s) == RLD_EINVAL);
  free(a);
  free(b);
  free(s);

  const uint32_t ids[3] = {2, 0, 2};
  const uint64_t aa[3] = {0x10, 0x20, 0x30}, bb[3] = {0x40, 0x50, 0x60};
  const float sc[3] = {1.f, 2.f, 3.f};
  uint64_t* ao = (uint64_t*)malloc(sizeof(uint64_t) * 3);
  uint64_t* bo = (uint64_t*)malloc(sizeof(uint64_t) * 3);
  float* so = (float*)malloc(sizeof(float) * 3);
  uint32_t n = 99;
  EXPECT(rld_pack_expert_tables(ids, aa, bb, sc, 3, 3, ao, bo, so, &n) == RLD_OK && n == 3);
  EXPECT(ao[2] == 0x30 && so[2] == 3.f && ao[1] == 0 && ao[0] == 0x20);
  EXPECT(rld_pack_expert_tables(ids, aa, bb, sc, 3, 2, ao, bo, so, &n) == RLD_ENOSPACE);
  EXPECT(rld_pack_expert_tables(ids, aa, bb, sc, 0, 0, nullptr, nullptr, nullptr, &n) == RLD_OK &&
         n == 0);
  const uint32_t big[1] = {0xFFFFFFFFu};  // n = 2^32 cannot fit any cap
  EXPECT(rld_pack_expert_tables(big, aa, bb, sc, 1, 0xFFFFFFFFu, ao, bo, so, &n) ==
         RLD_ENOSPACE);
  free(ao);
  free(bo);
  free(so);
}

static void check_windows() {
  struct Case {
    uint32_t total, cap, count;
  } cases[] = {{0, 8192, 0},           {1, 8192, 1},          {32768, 8192, 4},
               {32769, 8192, 5},       {0xFFFFFFFFu, 0x80000000u, 2},
               {0xFFFFFFFFu, 0xFFFFFFFFu, 1}, {0xFFFFFFFEu, 0x7FFFFFFFu, 2},
               {0xFFFFFFFFu, 0x10000000u, 16}};
  for (const Case& c : cases) {
    uint32_t* st = (uint32_t*)malloc(sizeof(uint32_t) * (c.count ? c.count : 1));
    uint32_t* en = (uint32_t*)malloc(sizeof(uint32_t) * (c.count ? c.count : 1));
    uint32_t n = 99;
    EXPECT(rld_grouped_windows(c.total, c.cap, st, en, c.count, &n) == RLD_OK && n == c.count);
    for (uint32_t k = 0; k < n; ++k) {
      EXPECT(st[k] == k * c.cap);
      EXPECT(en[k] == (k + 1 == n ? c.total : (k + 1) * c.cap));
    }
    if (c.count > 0)
      EXPECT(rld_grouped_windows(c.total, c.cap, st, en, c.count - 1, &n) == RLD_ENOSPACE);
    free(st);
    free(en);
  }
  uint32_t n = 0;
  EXPECT(rld_grouped_windows(10, 0, nullptr, nullptr, 0, &n) == RLD_EINVAL);
  EXPECT(rld_grouped_wc(0, 0) == 1 && rld_grouped_wc(0, 65) == 2 && rld_grouped_wc(9, 3) == 0);
  EXPECT(rld_grouped_wc(0, 0xFFFFFFFFu) == 0x4000000u);
  EXPECT(rld_gather_row_token(17, 8) == 2 && rld_gather_row_token(5, 0) == 0);
  uint32_t g[12];
  EXPECT(rld_gather_grids(16, 0xFFFFFFFFu, 256, g) == RLD_OK && g[0] == 256 &&
         g[7] == 0x800000u);
  EXPECT(rld_gather_grids(16, 2048, 256, nullptr) == RLD_EINVAL);
}

static void check_status() {
  for (int st = 1; st >= -6; --st) EXPECT(rld_status_string(st) != nullptr);
  EXPECT(rld_version() != nullptr && rld_last_hip_error() == 0);
}

int main() {
  check_scale();
  check_f16();
  check_pad();
  check_route_pack();
  check_moe_pack();
  check_windows();
  check_status();
  if (g_fail) {
    fprintf(stderr, "%d failed\n", g_fail);
    return 1;
  }
  printf("ok\n");
  return 0;
}
