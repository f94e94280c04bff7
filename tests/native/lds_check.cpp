// lds_check.cpp -- host check of the LDS reservations every context launches
// with (sharded_optimizer_step_zero_amd/csrc/lds.h): every table entry and every
// ZS_WAVES_PER_CU value gives reservations that fit a 64 KiB per-workgroup
// limit with room for the kernels' static LDS and reach the intended residency;
// the init-time check refuses a plan that does not fit; the override parser
// takes exactly the documented values.  Built with g++ and run by
// tests/test_lds_reservations.py (no GPU).
#include <stdio.h>

#include <initializer_list>

#include "../../sharded_optimizer_step_zero_amd/csrc/lds.h"

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      failures++;                                                         \
    }                                                                     \
  } while (0)

using namespace zs;

// The smallest per-workgroup LDS limit among CDNA parts, and room for static LDS.
constexpr size_t kWgLimit = 64 * 1024;
constexpr size_t kStaticRoom = 256;

static void check_reservation(int32_t per_cu, size_t lds_cu, bool exact) {
  const size_t r = lds_reservation(per_cu, lds_cu);
  if (per_cu <= 0) {
    CHECK(r == 0);
    return;
  }
  CHECK(r > 0 && r % 256 == 0);
  CHECK(r + kStaticRoom <= kWgLimit);
  const size_t fit = lds_cu / r;           // workgroups that reside together
  CHECK(fit >= (size_t)per_cu);            // never fewer than asked for
  if (exact) CHECK(fit == (size_t)per_cu); // the measured caps are met exactly
}

int main() {
  const size_t lds_cu = kLdsPerCuDefault;
  // every entry of the step, staged-norm and copy tables
  for (int M = 1; M <= kCapMaxM; M++) {
    check_reservation(kStepWavesSmall[M], lds_cu, true);
    check_reservation(kStepWavesLarge[M], lds_cu, true);
    check_reservation(kStepWavesHuge[M], lds_cu, true);
    check_reservation(kStageWgsPerCu[M], lds_cu, true);
    CHECK(kStepWavesSmall[M] >= kMinWavesPerCu && kStepWavesLarge[M] >= kMinWavesPerCu &&
          kStepWavesHuge[M] >= kMinWavesPerCu);
  }
  check_reservation(kCopyWavesPerCu, lds_cu, true);
  // the one-round rule never asks for more than 16 waves per CU
  for (int M = 1; M <= kCapMaxM; M++)
    for (int64_t n : {int64_t(0), int64_t(256), int64_t(1) << 20, int64_t(3) << 20,
                      int64_t(1) << 28})
      for (int32_t cu : {1, 80, 256, 304}) {
        const int32_t w = step_waves_per_cu(M, n, cu, kWavesFromTable);
        CHECK(w >= kMinWavesPerCu && w <= 16);
        check_reservation(w, lds_cu, true);
      }
  // every override value, every M, every size column, the whole plan
  const int64_t sizes[] = {0, 1, 1 << 20, (int64_t(1) << 28) + 1, (int64_t(1) << 31) + 1,
                           int64_t(1) << 34};
  for (int32_t ov = kWavesFromTable; ov <= kMaxWavesPerCu; ov++) {
    if (ov == 1 || ov == 2) continue;  // not accepted (parser below)
    for (int M = 1; M <= kCapMaxM; M++)
      for (int64_t n : sizes) {
        const LdsPlan p = lds_plan(M, n, 256, lds_cu, ov);
        const int32_t w = step_waves_per_cu(M, n, 256, ov);
        if (ov >= 0) CHECK(w == ov);
        check_reservation(w, lds_cu, ov <= 24);  // 256-byte units make caps above 24 approximate
        CHECK(lds_plan_fits(p, kStaticRoom, kWgLimit, lds_cu));
        CHECK(p.copy == lds_reservation(kCopyWavesPerCu, lds_cu));
        CHECK(p.stage_norm == lds_reservation(kStageWgsPerCu[M], lds_cu));
      }
  }
  // the init-time check refuses what does not fit
  {
    const LdsPlan p3 = lds_plan(8, 1 << 20, 256, lds_cu, 3);  // 54,528 B per workgroup
    CHECK(p3.step == 54528);
    CHECK(lds_plan_fits(p3, 32, kWgLimit, lds_cu));
    CHECK(!lds_plan_fits(p3, 32, 48 * 1024, lds_cu));          // a smaller per-workgroup limit
    CHECK(!lds_plan_fits(p3, 11 * 1024, kWgLimit, lds_cu));     // static LDS pushes it over
    CHECK(!lds_plan_fits(p3, 32, kWgLimit, 32 * 1024));         // less LDS per CU
    const LdsPlan p0 = lds_plan(2, 1 << 20, 256, lds_cu, 0);    // uncapped steps, M = 2
    CHECK(p0.step == 0 && p0.step_staged == 0 && p0.stage_norm == 0 && p0.copy > 0);
    CHECK(lds_plan_fits(p0, 32, p0.copy + 32, lds_cu));
    CHECK(!lds_plan_fits(p0, 32, p0.copy + 31, lds_cu));
  }
  // the override parser
  {
    int32_t v = 123;
    CHECK(parse_waves_override(nullptr, &v) && v == kWavesFromTable);
    CHECK(parse_waves_override("", &v) && v == kWavesFromTable);
    CHECK(parse_waves_override("0", &v) && v == 0);
    CHECK(parse_waves_override("3", &v) && v == 3);
    CHECK(parse_waves_override("64", &v) && v == 64);
    for (const char* bad : {"1", "2", "65", "-1", "-3", "abc", "7x", "9.5", " "})
      CHECK(!parse_waves_override(bad, &v));
  }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("lds check ok\n");
  return 0;
}
