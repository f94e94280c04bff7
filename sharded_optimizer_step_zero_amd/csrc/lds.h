// lds.h -- resident-workgroup caps of the streaming kernels and the LDS
// reservations that impose them, with the check every context runs at init.
//
// A streaming kernel here touches no LDS for its data; its launch asks for a
// dynamic LDS block it never uses, sized so that at most `per_cu` workgroups
// fit on a CU at once.  That caps the bytes each CU keeps in flight, which is
// what the measured caps below tune.  The request (dynamic + the kernel's own
// static LDS) must stay within the device's per-workgroup limit, or the launch
// fails or misbehaves, so a context computes every reservation it will use
// once, at init, against the limits queried from the device, and refuses to
// start when one does not fit.
//
// Host-only arithmetic (no HIP calls), shared by the C ABI and its CPU tests.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

namespace zs {

// LDS per CU on gfx950 (used when the device query fails).
constexpr size_t kLdsPerCuDefault = 160 * 1024;
// Per-workgroup LDS limit assumed when the device reports none: the smallest
// among CDNA parts (MI355X reports 160 KiB).
constexpr size_t kLdsPerWorkgroupFallback = 64 * 1024;
constexpr int kCapMaxM = 16;
// The smallest cap that can be asked for: below 3 resident waves per CU the
// reservation would exceed what one workgroup may hold on CDNA parts with a
// 64 KiB per-workgroup limit, so caps 1 and 2 are not offered.
constexpr int32_t kMinWavesPerCu = 3;
constexpr int32_t kMaxWavesPerCu = 64;

// Resident-wave cap of the step kernels per CU, by M and shard size (three
// columns: up to 2^28 elements, up to 2^31, above).  Measured on MI355X with
// the device-scope non-temporal stores and the staggered slab placement: caps
// 5..12 swept for every M on flat 164M-, 1G- and 4.3G-element shards, two
// rounds on the same buffers (repeatable to 0.3%), and checked on the GPT,
// Llama and stress layouts.  Fewer contributions leave each wave less in
// flight, so more waves pay off; from M = 10 on, 7 waves are best everywhere (6
// and 5 lose 3-20%).  Re-measured on the Llama-70B 1/16 shard (M = 8, above
// 2^31), caps 5-12 on the same buffers in four allocations on two boxes: 8 and
// 9 tied 7 or led it by up to 1.3% in three, trailed by 0.6% in one, so that
// entry is 8.
//                                                 M: 0   1   2   3   4   5  6  7  8  9 10 11 12 13 14 15 16
constexpr int8_t kStepWavesSmall[kCapMaxM + 1] = {0, 12, 11, 11, 10, 10, 9, 9, 9, 9, 7, 7, 7, 7, 7, 7, 7};
constexpr int8_t kStepWavesLarge[kCapMaxM + 1] = {0, 11, 11, 10, 9, 9, 8, 8, 8, 8, 7, 7, 7, 7, 7, 7, 7};
constexpr int8_t kStepWavesHuge[kCapMaxM + 1] = {0, 12, 10, 10, 8, 8, 9, 9, 8, 7, 7, 7, 7, 7, 7, 7, 7};

// Resident workgroups per CU of the staged norm pass (0: no cap), by M.  The
// staged pass adds a write stream to a read pass; the more contributions each
// workgroup reads, the fewer of them stream best.  Measured on MI355X
// (GPT-1.3B-size shard, the loss-scaled and the clipped bf16 step, same
// buffers): M = 2 uncapped; M = 4: 6 (-2.1% step time); M = 8: 5 (-3.4%);
// M = 16: 4 (-2.6%).  The fused (read-only) pass runs uncapped: caps measured
// neutral to slower there.
constexpr int8_t kStageWgsPerCu[kCapMaxM + 1] = {0, 0, 0, 6, 6, 5, 5, 5, 5, 4, 4, 4, 4, 4, 4, 4, 4};

// Resident single-wave workgroups per CU of the state export/import copy
// (caps 9-14 swept on the GPT-1.3B shard; 10 was best).
constexpr int32_t kCopyWavesPerCu = 10;

// Step-kernel tiles, elements (one single-wave workgroup each).
constexpr int64_t kCapTileElems = 256;

// No override: the step kernels take the measured table.
constexpr int32_t kWavesFromTable = -1;

// The step kernels' cap for M contributions over a shard, on n_cu CUs (0: no
// cap).  override_waves: kWavesFromTable uses the table; 0 (no cap) or
// kMinWavesPerCu..kMaxWavesPerCu replaces it.
inline int32_t step_waves_per_cu(int32_t M, int64_t shard_len, int32_t n_cu,
                                 int32_t override_waves) {
  if (M < 1 || M > kCapMaxM) return 0;
  if (override_waves != kWavesFromTable) return override_waves;
  int32_t cap;
  if (shard_len <= (int64_t(1) << 28)) cap = kStepWavesSmall[M];
  else cap = shard_len <= (int64_t(1) << 31) ? kStepWavesLarge[M] : kStepWavesHuge[M];
  // A grid that up to 16 waves per CU cover in one round runs as one round: at
  // 1M elements (4,096 tiles) the table's cap leaves a partial second round,
  // and cap 16 measured 0-14% faster there (M = 1..16); smaller grids keep the
  // table's cap, which spreads their few waves over more CUs.
  if (n_cu < 1) n_cu = 1;
  const int64_t tiles = (shard_len + kCapTileElems - 1) / kCapTileElems;
  const int64_t one_round = (tiles + n_cu - 1) / n_cu;
  if (one_round > cap && one_round <= 16) cap = (int32_t)one_round;
  return cap;
}

// The dynamic LDS a workgroup asks for so that at most per_cu of them reside on
// a CU with lds_per_cu bytes (0: no cap), in whole 256-byte allocation units.
inline size_t lds_reservation(int32_t per_cu, size_t lds_per_cu) {
  if (per_cu <= 0) return 0;
  return (lds_per_cu / (size_t)per_cu) & ~(size_t)255;
}

// Parses a ZS_WAVES_PER_CU value: unset or empty (kWavesFromTable), 0 (no
// cap) or kMinWavesPerCu..kMaxWavesPerCu.  Returns false for anything else
// (text, negative values, 1, 2, beyond 64).
inline bool parse_waves_override(const char* s, int32_t* out) {
  *out = kWavesFromTable;
  if (!s || !*s) return true;
  char* end = nullptr;
  const long v = strtol(s, &end, 10);
  if (*end != '\0') return false;
  if (v != 0 && (v < kMinWavesPerCu || v > kMaxWavesPerCu)) return false;
  *out = (int32_t)v;
  return true;
}

// Every dynamic LDS reservation a context launches with.
struct LdsPlan {
  size_t step;         // the fused bf16 and fp16 step kernels
  size_t step_staged;  // the step on staged averages
  size_t stage_norm;   // the staged norm passes
  size_t copy;         // state export/import
};

inline LdsPlan lds_plan(int32_t M, int64_t shard_len, int32_t n_cu, size_t lds_per_cu,
                        int32_t override_waves) {
  LdsPlan p;
  p.step = lds_reservation(step_waves_per_cu(M, shard_len, n_cu, override_waves), lds_per_cu);
  // the staged step reads 16 B of gradient per lane, as many bytes as M = 2
  p.step_staged =
      lds_reservation(step_waves_per_cu(2, shard_len, n_cu, override_waves), lds_per_cu);
  p.stage_norm = (M >= 1 && M <= kCapMaxM) ? lds_reservation(kStageWgsPerCu[M], lds_per_cu) : 0;
  p.copy = lds_reservation(kCopyWavesPerCu, lds_per_cu);
  return p;
}

// True when every reservation plus the largest static LDS of the kernels that
// take it fits the device's per-workgroup limit and its LDS per CU.
inline bool lds_plan_fits(const LdsPlan& p, size_t max_static, size_t per_wg_limit,
                          size_t lds_per_cu) {
  const size_t r[4] = {p.step, p.step_staged, p.stage_norm, p.copy};
  for (size_t x : r) {
    if (x == 0) continue;
    if (x + max_static > per_wg_limit || x + max_static > lds_per_cu) return false;
  }
  return true;
}

}  // namespace zs
