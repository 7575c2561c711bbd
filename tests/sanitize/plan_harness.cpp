// Host-only check of the decode library's launch-plan and workspace arithmetic
// (plan.h, compiled as plain C++ with -fsanitize=address,undefined): every
// shape and budget the C ABI accepts is planned and its invariants checked.
// Exit status 0 = all invariants hold; the sanitizers abort on any overflow or
// out-of-bounds access in the arithmetic.
#include <stdint.h>
#include <stdio.h>

#include "plan.h"

using adamas::Plan;

static int failures = 0;
static long checked = 0;

#define REQUIRE(cond, ...)                                          \
  do {                                                              \
    if (!(cond)) {                                                  \
      if (failures < 20) {                                          \
        printf("FAIL %s: ", #cond);                                 \
        printf(__VA_ARGS__);                                        \
        printf("\n");                                               \
      }                                                             \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static void check(int B, int Hq, int Hkv, int cap, int budget, bool dense) {
  const Plan p = adamas::make_plan(B, Hq, Hkv, cap, budget, dense);
  ++checked;
  const char* fmt = "B=%d Hq=%d Hkv=%d cap=%d budget=%d dense=%d";
#define ARGS B, Hq, Hkv, cap, budget, (int)dense
  REQUIRE(p.total > 0 && p.total % 256 == 0, fmt, ARGS);
  REQUIRE(p.total < ((size_t)1 << 42), fmt, ARGS);
  REQUIRE((int64_t)p.nch * p.chunk >= cap && p.chunk > 0 && (p.chunk & (p.chunk - 1)) == 0, fmt, ARGS);
  REQUIRE(p.off_part % 256 == 0 && p.off_count % 256 == 0 && p.off_count >= p.off_part && p.total > p.off_count,
          fmt, ARGS);
  if (dense) return;
  REQUIRE(p.off_sorted % 256 == 0 && p.off_rec % 256 == 0 && p.off_rec > p.off_sorted && p.off_part > p.off_rec,
          fmt, ARGS);
  REQUIRE(p.off_sync == 0 && p.off_sorted >= adamas::kSyncBytes, fmt, ARGS);  // sync words at a fixed place
  if (p.fused)  // single launch: groups and chunks within the sync words, a block per (head, split)
    REQUIRE((int64_t)B * Hkv <= adamas::kFusedMaxGroups && p.nch <= adamas::kFusedMaxChunks &&
                p.R * p.splits <= p.nch,
            fmt, ARGS);
  // every region holds what the kernels index in it
  const size_t bhq = (size_t)B * Hq;
  REQUIRE(p.off_rec - p.off_sorted >= bhq * p.nch * (size_t)p.chunk * sizeof(uint16_t), fmt, ARGS);
  REQUIRE(p.off_part - p.off_rec >= bhq * p.nch * (size_t)adamas::kRecStride * sizeof(uint16_t), fmt, ARGS);
  REQUIRE(p.off_count - p.off_part >= bhq * p.splits * (size_t)adamas::kPartFloats * sizeof(float), fmt, ARGS);
  REQUIRE(p.total - p.off_count >= bhq * sizeof(uint32_t), fmt, ARGS);
  if (!p.supported) return;
  const int kb = budget < cap ? budget : cap;
  REQUIRE(p.splits >= 1 && p.rows_per_split >= 1 && p.rows_per_split % 128 == 0, fmt, ARGS);
  REQUIRE((int64_t)p.splits * p.rows_per_split >= kb, fmt, ARGS);
  REQUIRE((int64_t)(p.splits - 1) * p.rows_per_split < kb, fmt, ARGS);  // no empty split
  REQUIRE(p.lds_select <= adamas::kSelectDynLdsMax, fmt, ARGS);
  REQUIRE(p.nch <= adamas::kSelMaxChunks, fmt, ARGS);
#undef ARGS
}

// div_by against the plain division: small divisors with every numerator
// below 2^16, then divisors and numerators up to 2^31 - 1 near the points
// where the estimate can fall one short (multiples of d, and their neighbours)
static long divisions = 0;
static void check_division() {
  for (int d = 1; d <= 600; ++d) {
    const uint32_t m = adamas::div_magic(d);
    for (int n = 0; n < 65536; ++n, ++divisions) REQUIRE(adamas::div_by(n, d, m) == n / d, "n=%d d=%d", n, d);
  }
  const int ds[] = {601, 1000, 4095, 4096, 4097, 65535, 65536, 65537, 1 << 20, 1000003, (1 << 30) - 1, 1 << 30,
                    2147483646, 2147483647};
  for (int d : ds) {
    const uint32_t m = adamas::div_magic(d);
    for (int64_t k = 0; k * d <= 2147483647 && k < 100000; k += 1 + k / 64) {
      for (int64_t delta = -2; delta <= 2; ++delta) {
        const int64_t n = k * d + delta;
        if (n < 0 || n > 2147483647) continue;
        REQUIRE(adamas::div_by((int)n, d, m) == (int)(n / d), "n=%lld d=%d", (long long)n, d);
        ++divisions;
      }
    }
    const int ns[] = {0, 1, 2147483646, 2147483647};
    for (int n : ns) REQUIRE(adamas::div_by(n, d, m) == n / d, "n=%d d=%d", n, d);
  }
}

int main() {
  check_division();
  const int caps[] = {1, 2, 5, 63, 64, 65, 127, 511, 512, 513, 1000, 4095, 4096, 4097, 16384, 32768, 65536,
                      131072, 262144, 524287, 524288};
  const int budgets[] = {1, 2, 7, 16, 63, 64, 65, 127, 128, 129, 255, 256, 700, 1023, 1024, 1025, 4096, 5000,
                         8192, 65536, 229376, 229377, 1 << 20, (1 << 30) + 7, 2147483646, 2147483647};
  const int shapes[][3] = {{1, 1, 1}, {1, 8, 1}, {1, 32, 8}, {2, 32, 8}, {16, 32, 8}, {3, 6, 3},
                           {1024, 32, 8}, {2048, 32, 8}, {65535, 1, 1}, {8191, 8, 1}};
  for (const auto& s : shapes) {
    for (int cap : caps) {
      if ((int64_t)s[0] * s[1] * cap > ((int64_t)1 << 33)) continue;  // (beyond any device's memory)
      check(s[0], s[1], s[2], cap, 1, true);
      for (int budget : budgets) check(s[0], s[1], s[2], cap, budget, false);
      check(s[0], s[1], s[2], cap, cap, false);
      if (cap < (1 << 30)) check(s[0], s[1], s[2], cap, 2 * cap, false);
    }
  }
  printf("divisions checked: %ld\n", divisions);
  printf("plan checks: %ld, failures: %d\n", checked, failures);
  return failures ? 1 : 0;
}
