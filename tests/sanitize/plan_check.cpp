// plan_check.cpp -- the layout planner (plan.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: plans for many seeded tensor lists (zero-size
// tensors, tensors above the bucket cap, alignments 1..128, 1..16 ranks, every
// rank) through the public C functions, with the layout's invariants checked:
// segments and runs partition [0, shard_len) in order, padding is where no
// tensor is, every tensor element lands on exactly one rank, bucket lengths are
// non-zero multiples of world_size * align, the per-stage byte counts follow
// their formulas, and the export/import piece table (internal to the planner)
// covers every owned tensor element exactly once with consistent canonical
// offsets: whole pieces of kPieceElems elements first, then parts of at most
// kCopyPart.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <string>
#include <vector>

#include "../../include/zeroshard.h"
#include "../../sharded_optimizer_step_zero_amd/csrc/internal.h"

namespace zs {
void set_error(const std::string&) {}
}  // namespace zs

static uint64_t rng = 0x243F6A8885A308D3ull;
static uint64_t next_u64() {  // xorshift64* (inputs only)
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return rng * 0x2545F4914F6CDD1Dull;
}

#define REQUIRE(c)                                                        \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                           \
    }                                                                     \
  } while (0)

// The piece table: sizes by kind, each piece inside one tensor segment with the
// canonical offset of its first element, and together an exact cover of the
// shard's tensor elements.
static int check_pieces(const zs_plan* p, const std::vector<int64_t>& numel) {
  std::vector<int64_t> canon(numel.size(), 0);
  for (size_t t = 1; t < numel.size(); t++) canon[t] = canon[t - 1] + numel[t - 1];
  const int64_t nw = p->n_whole_pieces;
  REQUIRE(nw >= 0 && nw <= (int64_t)p->pieces.size());
  int64_t owned = 0;
  for (const zs::Segment& sg : p->segments)
    if (sg.tensor >= 0) owned += sg.len;
  std::vector<std::pair<int64_t, int64_t>> spans;
  int64_t sum = 0;
  for (size_t i = 0; i < p->pieces.size(); i++) {
    const zs::Piece& pc = p->pieces[i];
    if ((int64_t)i < nw) REQUIRE(pc.len == zs::kPieceElems);
    else REQUIRE(pc.len >= 1 && pc.len <= zs::kCopyPart);
    // the segment holding the piece's first element
    const zs::Segment* seg = nullptr;
    for (const zs::Segment& sg : p->segments)
      if (sg.shard_off <= pc.shard_off && pc.shard_off < sg.shard_off + sg.len) seg = &sg;
    REQUIRE(seg && seg->tensor >= 0);
    REQUIRE(pc.shard_off + pc.len <= seg->shard_off + seg->len);
    REQUIRE(pc.canon_off == canon[seg->tensor] + seg->tensor_off + (pc.shard_off - seg->shard_off));
    spans.push_back({pc.shard_off, pc.len});
    sum += pc.len;
  }
  REQUIRE(sum == owned);
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); i++)
    REQUIRE(spans[i - 1].first + spans[i - 1].second <= spans[i].first);
  return 0;
}

static int check_layout(const std::vector<int64_t>& numel, const std::vector<uint8_t>& decay,
                        int32_t N, int64_t cap, int32_t align) {
  int64_t total = 0;
  for (int64_t n : numel) total += n;
  std::vector<int64_t> covered(numel.size(), 0);
  int64_t padded_prev = -1;
  for (int32_t r = 0; r < N; r++) {
    zs_plan* raw = nullptr;
    REQUIRE(zs_plan_create(numel.data(), decay.data(), (int64_t)numel.size(), N, r, cap, align,
                           &raw) == ZS_OK);
    std::unique_ptr<zs_plan, void (*)(zs_plan*)> owner(raw, zs_plan_destroy);
    const zs_plan* p = raw;
    int64_t S, nseg, nruns, padded, nb;
    REQUIRE(zs_plan_query(p, &S, &nseg, &nruns, &padded, &nb) == ZS_OK);
    REQUIRE(padded_prev < 0 || padded == padded_prev);
    padded_prev = padded;
    REQUIRE(S * N == padded);
    int64_t sum_b = 0;
    for (int64_t b = 0; b < nb; b++) {
      int64_t off, len;
      REQUIRE(zs_plan_bucket(p, b, &off, &len) == ZS_OK);
      // no bucket is empty unless the whole model is
      REQUIRE(off == sum_b && len % ((int64_t)N * align) == 0 && (len > 0 || total == 0));
      sum_b += len;
    }
    REQUIRE(sum_b == padded);
    int64_t pos = 0;
    for (int64_t s = 0; s < nseg; s++) {
      int64_t off, len, t, toff;
      int32_t dec;
      REQUIRE(zs_plan_segment(p, s, &off, &len, &t, &toff, &dec) == ZS_OK);
      REQUIRE(off == pos && len > 0);
      if (t >= 0) {
        REQUIRE(t < (int64_t)numel.size() && toff >= 0 && toff + len <= numel[t]);
        REQUIRE(dec == (decay[t] ? 1 : 0));
        covered[t] += len;
        int64_t so, to, l;
        REQUIRE(zs_plan_tensor_slice(p, t, &so, &to, &l) == ZS_OK);
        REQUIRE(so == off && to == toff && l == len);
      } else {
        REQUIRE(dec == 0);
      }
      pos += len;
    }
    REQUIRE(pos == S);
    int64_t rpos = 0;
    for (int64_t i = 0; i < nruns; i++) {
      int64_t start, len;
      int32_t flags;
      REQUIRE(zs_plan_run(p, i, &start, &len, &flags) == ZS_OK);
      REQUIRE(start == rpos && len > 0);
      rpos += len;
    }
    REQUIRE(rpos == S);
    int64_t b0, b1, b2, b3;
    REQUIRE(zs_plan_state_bytes(p, 0, &b0) == ZS_OK && b0 == 16 * total);
    REQUIRE(zs_plan_state_bytes(p, 1, &b1) == ZS_OK && b1 == 4 * total + 12 * S);
    REQUIRE(zs_plan_state_bytes(p, 2, &b2) == ZS_OK && b2 == 2 * total + 14 * S);
    REQUIRE(zs_plan_state_bytes(p, 3, &b3) == ZS_OK && b3 == 16 * S);
    int64_t x;
    REQUIRE(zs_plan_segment(p, nseg, &x, &x, &x, &x, nullptr) == ZS_EINVAL);
    REQUIRE(check_pieces(p, numel) == 0);
  }
  for (size_t t = 0; t < numel.size(); t++) REQUIRE(covered[t] == numel[t]);
  return 0;
}

int main() {
  int cases = 0;
  const int32_t aligns[] = {8, 16, 64, 128, 8};
  for (int it = 0; it < 60; it++) {
    const int n = 1 + (int)(next_u64() % 40);
    std::vector<int64_t> numel(n);
    std::vector<uint8_t> decay(n);
    for (int i = 0; i < n; i++) {
      const uint64_t k = next_u64() % 10;
      numel[i] = k == 0 ? 0 : (k < 8 ? (int64_t)(next_u64() % 5000) : (int64_t)(next_u64() % 300000));
      decay[i] = (uint8_t)(next_u64() & 1);
    }
    const int32_t N = 1 + (int32_t)(next_u64() % 16);
    const int64_t cap = 1000 + (int64_t)(next_u64() % 200000);
    const int32_t align = aligns[next_u64() % 5];
    if (check_layout(numel, decay, N, cap, align)) {
      fprintf(stderr, "case %d: n=%d N=%d cap=%lld align=%d\n", it, n, N, (long long)cap, align);
      return 1;
    }
    cases++;
  }
  // argument errors are reported, not crashed on
  zs_plan* p = nullptr;
  const int64_t one = 10;
  const uint8_t d1 = 1;
  if (zs_plan_create(&one, &d1, 1, 2, 2, 100, 64, &p) != ZS_EINVAL) return 1;
  if (zs_plan_create(&one, &d1, 1, 1, 0, 100, 0, &p) != ZS_EINVAL) return 1;
  if (zs_plan_create(&one, &d1, 1, 1, 0, 100, 1, &p) != ZS_EINVAL) return 1;  // align must be a multiple of 8
  if (zs_plan_create(nullptr, nullptr, 0, 3, 1, 100, 64, &p) != ZS_OK) return 1;
  zs_plan_destroy(p);
  printf("plan check ok: %d layouts over every rank\n", cases);
  return 0;
}
