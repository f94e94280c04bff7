// plan.cpp -- the flat bucket / shard layout and the weight-decay runs of a shard.
//
// Layout (integer work, once per model):
//  1. Tensors are placed in forward order into buckets, each at the next
//     multiple of `align` elements from its bucket's start; a bucket closes
//     when the next tensor would end past `bucket_cap`; a larger tensor sits
//     alone; a bucket closes only once it holds elements, and a tensor with
//     no elements never closes one, so no bucket is left empty (gradient
//     buckets: 大模型基础设施工程 06, §6.1; contiguous flat
//     gradient buffers: same page, §11.3).
//  2. A bucket's length is padded to a multiple of world_size * align, so
//     its world_size slices are equal and aligned ("padded to the shard
//     boundary").
//  3. Rank r owns slice r of every bucket: the part of the reduced gradient a
//     reduce-scatter leaves on it and the only part it updates (Lecture04
//     notes, "ZeRO-1"; CS324 notes §3.4).  Its shard concatenates those
//     slices in bucket order; flat cutting is legal because AdamW is
//     elementwise (CS324 notes §3.4).
//  4. Segments are maximal runs of one tensor or of padding in the shard.
//  5. Runs: maximal stretches of the shard with one weight-decay flag; padding
//     joins the run it follows (or the next one at the shard's start) -- it is
//     zero in every array and stays zero under either flag.  Every run start
//     is a tensor start, hence a multiple of `align`.  The step kernel tiles
//     the flat shard uniformly and looks each tile's flag up in this table,
//     so thousands of mixed-size tensors cost one launch and a short search.
//  6. Pieces: the tensor segments again, with their offsets in the canonical
//     order (every tensor contiguous and unpadded, in forward order) -- the
//     format a checkpoint stores, independent of N and of the bucket layout.
//     The table lists every whole piece (kPieceElems elements) first, then the
//     rest of each segment cut into parts of at most kCopyPart elements, so
//     the copy kernel runs exactly one work-group per part.
#include <string.h>

#include <algorithm>
#include <new>

#include "../../include/zeroshard.h"
#include "internal.h"

namespace zs {
void set_error(const std::string& msg);
}

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 52;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int fail(const char* msg) {
  zs::set_error(msg);
  return ZS_EINVAL;
}

void build_runs(zs_plan& p) {
  p.runs.clear();
  int last_flag = -1;  // flag of the open run; -1 while it holds only padding
  for (const zs::Segment& s : p.segments) {
    if (s.tensor < 0) {  // padding joins the current run
      if (p.runs.empty()) p.runs.push_back({s.shard_off, 0, 0});
      continue;
    }
    if (!p.runs.empty() && (last_flag == -1 || last_flag == s.decay)) {
      p.runs.back().flags = s.decay;
    } else {
      p.runs.push_back({s.shard_off, s.decay, 0});
    }
    last_flag = s.decay;
  }
}

// The run table as the step kernels read it (the runs, at least one, then a
// sentinel starting past the shard) and, with more than one run, the tile-flag
// table: per 256-element tile, 2 bits -- the decay flag of a tile inside one
// run, or 2 for a tile that straddles a run boundary.
void build_step_tables(zs_plan& p) {
  p.run_table = p.runs;
  if (p.run_table.empty()) p.run_table.push_back({0, 0, 0});
  p.run_table.push_back({p.shard_len, 0, 0});
  const int64_t n_runs = (int64_t)p.run_table.size() - 1;
  p.tile_flags.assign((size_t)zs::tile_flag_words(p.shard_len, n_runs), 0u);
  if (p.tile_flags.empty()) return;
  const int64_t tiles = (p.shard_len + zs::kStepTileElems - 1) / zs::kStepTileElems;
  size_t r = 0;  // the run holding the tile's first element
  for (int64_t t = 0; t < tiles; t++) {
    const int64_t lo = t * zs::kStepTileElems;
    const int64_t hi = std::min(p.shard_len, lo + zs::kStepTileElems);
    while (p.run_table[r + 1].start <= lo) r++;
    const uint32_t f = p.run_table[r + 1].start < hi ? 2u : (uint32_t)(p.run_table[r].flags & 1);
    p.tile_flags[(size_t)(t >> 4)] |= f << ((t & 15) * 2);
  }
}

}  // namespace

extern "C" int zs_plan_create(const int64_t* numel, const uint8_t* decay, int64_t n_tensors,
                              int32_t world_size, int32_t rank, int64_t bucket_cap,
                              int32_t align, zs_plan** out) {
  if (!out) return fail("zs_plan_create: out is NULL");
  *out = nullptr;
  if (n_tensors < 0 || (n_tensors > 0 && (!numel || !decay)))
    return fail("zs_plan_create: tensor arrays missing");
  if (world_size < 1 || rank < 0 || rank >= world_size)
    return fail("zs_plan_create: need 0 <= rank < world_size");
  if (bucket_cap < 1) return fail("zs_plan_create: bucket_cap must be >= 1");
  if (align < 8 || align % 8 != 0 || align > (1 << 20))
    return fail("zs_plan_create: align must be a multiple of 8 (at most 2^20)");
  int64_t total = 0;
  for (int64_t t = 0; t < n_tensors; t++) {
    if (numel[t] < 0 || numel[t] > kMaxElems)
      return fail("zs_plan_create: tensor size out of range");
    total += numel[t];
    if (total > kMaxElems) return fail("zs_plan_create: total size out of range");
  }
  if ((int64_t)world_size * align > (int64_t(1) << 30))
    return fail("zs_plan_create: world_size * align too large");

  zs_plan* p = new (std::nothrow) zs_plan;
  if (!p) {
    zs::set_error("zs_plan_create: out of host memory");
    return ZS_ENOMEM;
  }
  try {
    p->world_size = world_size;
    p->rank = rank;
    p->align = align;
    p->bucket_cap = bucket_cap;
    p->numel.assign(numel, numel + n_tensors);
    p->decay.resize(n_tensors);
    for (int64_t t = 0; t < n_tensors; t++) p->decay[t] = decay[t] ? 1 : 0;
    p->total_params = total;
    p->tensor_flat_off.assign(n_tensors, 0);
    p->tensor_segment.assign(n_tensors, -1);

    // 1-2. buckets
    std::vector<int64_t> first_of_bucket;
    const int64_t pad_to = (int64_t)world_size * align;
    int64_t start = 0, fill = 0;
    bool open = false;
    for (int64_t t = 0; t < n_tensors; t++) {
      int64_t pos = align_up(fill, align);
      // only a bucket that holds elements closes, and only for a tensor that has
      // some: no bucket is ever left empty
      if (open && fill > 0 && numel[t] > 0 && pos + numel[t] > bucket_cap) {
        int64_t len = align_up(fill, pad_to);
        p->bucket_off.push_back(start);
        p->bucket_len.push_back(len);
        start += len;
        fill = 0;
        pos = 0;
        open = false;
      }
      if (!open) {
        first_of_bucket.push_back(t);
        open = true;
      }
      p->tensor_flat_off[t] = start + pos;
      fill = pos + numel[t];
    }
    if (open) {
      p->bucket_off.push_back(start);
      p->bucket_len.push_back(align_up(fill, pad_to));
    }
    const int64_t nb = (int64_t)p->bucket_off.size();
    p->padded_total = nb ? p->bucket_off[nb - 1] + p->bucket_len[nb - 1] : 0;

    // 3-4. this rank's slices, cut into segments
    int64_t shard = 0;
    for (int64_t b = 0; b < nb; b++) {
      const int64_t part = p->bucket_len[b] / world_size;
      const int64_t lo = p->bucket_off[b] + rank * part, hi = lo + part;
      const int64_t t_end = b + 1 < nb ? first_of_bucket[b + 1] : n_tensors;
      int64_t cursor = lo;
      auto pad = [&](int64_t a, int64_t e) {
        if (e <= a) return;
        if (!p->segments.empty() && p->segments.back().tensor < 0 &&
            p->segments.back().shard_off + p->segments.back().len == shard + (a - lo))
          p->segments.back().len += e - a;
        else
          p->segments.push_back({shard + (a - lo), e - a, -1, 0, 0});
      };
      for (int64_t t = first_of_bucket[b]; t < t_end; t++) {
        const int64_t a = std::max(p->tensor_flat_off[t], lo);
        const int64_t e = std::min(p->tensor_flat_off[t] + numel[t], hi);
        if (a >= e) continue;
        pad(cursor, a);
        p->tensor_segment[t] = (int64_t)p->segments.size();
        p->segments.push_back(
            {shard + (a - lo), e - a, t, a - p->tensor_flat_off[t], (int32_t)p->decay[t]});
        cursor = e;
      }
      pad(cursor, hi);
      shard += part;
    }
    p->shard_len = shard;

    // 5. weight-decay runs, and the step kernels' run and tile-flag tables
    build_runs(*p);
    build_step_tables(*p);

    // 6. pieces for state export/import, with their offsets in the canonical
    //    order: the whole kPieceElems-element pieces of every tensor segment,
    //    then each segment's remainder in parts of at most kCopyPart elements
    std::vector<int64_t> canon(n_tensors, 0);
    for (int64_t t = 1; t < n_tensors; t++) canon[t] = canon[t - 1] + numel[t - 1];
    for (const zs::Segment& s : p->segments) {
      if (s.tensor < 0) continue;
      for (int64_t o = 0; o + zs::kPieceElems <= s.len; o += zs::kPieceElems)
        p->pieces.push_back(
            {s.shard_off + o, canon[s.tensor] + s.tensor_off + o, (int32_t)zs::kPieceElems, 0});
    }
    p->n_whole_pieces = (int64_t)p->pieces.size();
    for (const zs::Segment& s : p->segments) {
      if (s.tensor < 0) continue;
      for (int64_t o = s.len / zs::kPieceElems * zs::kPieceElems; o < s.len; o += zs::kCopyPart) {
        const int64_t len = std::min(zs::kCopyPart, s.len - o);
        p->pieces.push_back({s.shard_off + o, canon[s.tensor] + s.tensor_off + o, (int32_t)len, 0});
      }
    }
  } catch (const std::bad_alloc&) {
    delete p;
    zs::set_error("zs_plan_create: out of host memory");
    return ZS_ENOMEM;
  }
  *out = p;
  return ZS_OK;
}

extern "C" int zs_plan_query(const zs_plan* p, int64_t* shard_len, int64_t* n_segments,
                             int64_t* n_runs, int64_t* padded_total, int64_t* n_buckets) {
  if (!p) return fail("zs_plan_query: plan is NULL");
  if (shard_len) *shard_len = p->shard_len;
  if (n_segments) *n_segments = (int64_t)p->segments.size();
  if (n_runs) *n_runs = (int64_t)p->runs.size();
  if (padded_total) *padded_total = p->padded_total;
  if (n_buckets) *n_buckets = (int64_t)p->bucket_off.size();
  return ZS_OK;
}

extern "C" int zs_plan_tensor_slice(const zs_plan* p, int64_t tensor, int64_t* shard_off,
                                    int64_t* tensor_off, int64_t* len) {
  if (!p || !shard_off || !tensor_off || !len) return fail("zs_plan_tensor_slice: NULL argument");
  if (tensor < 0 || tensor >= (int64_t)p->numel.size())
    return fail("zs_plan_tensor_slice: tensor index out of range");
  int64_t s = p->tensor_segment[tensor];
  if (s < 0) {
    *shard_off = *tensor_off = *len = 0;
  } else {
    *shard_off = p->segments[s].shard_off;
    *tensor_off = p->segments[s].tensor_off;
    *len = p->segments[s].len;
  }
  return ZS_OK;
}

extern "C" int zs_plan_segment(const zs_plan* p, int64_t i, int64_t* shard_off, int64_t* len,
                               int64_t* tensor, int64_t* tensor_off, int32_t* decay) {
  if (!p || !shard_off || !len || !tensor || !tensor_off || !decay)
    return fail("zs_plan_segment: NULL argument");
  if (i < 0 || i >= (int64_t)p->segments.size())
    return fail("zs_plan_segment: index out of range");
  const zs::Segment& s = p->segments[i];
  *shard_off = s.shard_off;
  *len = s.len;
  *tensor = s.tensor;
  *tensor_off = s.tensor_off;
  *decay = s.decay;
  return ZS_OK;
}

extern "C" int zs_plan_bucket(const zs_plan* p, int64_t b, int64_t* flat_off, int64_t* len) {
  if (!p || !flat_off || !len) return fail("zs_plan_bucket: NULL argument");
  if (b < 0 || b >= (int64_t)p->bucket_off.size())
    return fail("zs_plan_bucket: index out of range");
  *flat_off = p->bucket_off[b];
  *len = p->bucket_len[b];
  return ZS_OK;
}

extern "C" int zs_plan_run(const zs_plan* p, int64_t i, int64_t* shard_off, int64_t* len,
                           int32_t* decay) {
  if (!p || !shard_off || !len || !decay) return fail("zs_plan_run: NULL argument");
  if (i < 0 || i >= (int64_t)p->runs.size()) return fail("zs_plan_run: index out of range");
  const int64_t end = i + 1 < (int64_t)p->runs.size() ? p->runs[i + 1].start : p->shard_len;
  *shard_off = p->runs[i].start;
  *len = end - p->runs[i].start;
  *decay = p->runs[i].flags & 1;
  return ZS_OK;
}

extern "C" int zs_plan_state_bytes(const zs_plan* p, int32_t stage, int64_t* bytes) {
  if (!p || !bytes) return fail("zs_plan_state_bytes: NULL argument");
  const int64_t psi = p->total_params, S = p->shard_len;
  switch (stage) {
    case 0: *bytes = 16 * psi; break;           // plain data parallelism
    case 1: *bytes = 4 * psi + 12 * S; break;   // optimizer state sharded
    case 2: *bytes = 2 * psi + 14 * S; break;   // + gradients sharded
    case 3: *bytes = 16 * S; break;             // + parameters sharded
    default: return fail("zs_plan_state_bytes: stage must be 0..3");
  }
  return ZS_OK;
}

extern "C" void zs_plan_destroy(zs_plan* p) { delete p; }
