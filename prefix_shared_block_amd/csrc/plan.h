// plan.h -- segment planner and launch geometry, shared by host and device.
//
// PrefixSharing PR #50 ("设计简介", design summary) replaces the per-rollout
// prefix copy with a visibility rule on the flat-packed buffer and suggests
// describing it by rectangles rather than a dense mask.  The planner realises
// that: every workgroup derives its own work item from its block index and
// the segment offsets, so no mask and no work list is ever stored.
//
// Flat work item: a tile of at most `tile_tokens` query tokens that lies
// entirely inside the prefix or inside one rollout, stacked with the G query
// heads of one kv head.  Its keys are range r0 = [0, P) plus r1 = [o_i, q_end)
// for a rollout tile (the shared prefix and the rollout's own tokens), or
// r0 = [0, q_end) for a prefix tile; a row r only keeps keys c <= r.
//
// Paged work item (sglang PR #27382, "实现拆解"): one split of one request's
// prefix for one kv head; every draft row sees every prefix key.
//
// Enumeration order (the contract the bit-exact planner test checks):
//  flat : block b -> kv head b % Hkv, per-head item j = b / Hkv; per head the
//         rollout tiles come first (rollouts in order, each from its last
//         tile to its first), then the prefix tiles from last to first, then
//         idle slots.  Longer items therefore start first, and all blocks of
//         one kv head share b % 8 and so land on the same XCD (blocks are
//         dealt round-robin over the 8 XCDs), keeping that head's K/V tiles
//         in one L2.
//  paged: block b -> split b % n_splits, kv head (b / n_splits) % Hkv,
//         request b / (n_splits * Hkv).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PS_HD __host__ __device__ __forceinline__
#else
#define PS_HD inline
#endif

namespace psattn {

enum ItemKind : int32_t { kNone = 0, kFlatPrefix = 1, kFlatSuffix = 2, kPagedSplit = 3 };

struct Item {
  int32_t kind, h_kv, seg, q_begin, q_end, r0_begin, r0_end, r1_begin, r1_end, split;
};

PS_HD int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
PS_HD int32_t cdiv32(int32_t a, int32_t b) { return (a + b - 1) / b; }
PS_HD int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }
PS_HD int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }

// ---------------------------------------------------------------- geometry
// Every prefix-pass workgroup is 4 waves of 64 lanes; each wave owns 32
// stacked query rows (one 32x32 MFMA column block).
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWaveRows = 32;

struct FlatGeom {
  int32_t rows;         // stacked rows per workgroup (128)
  int32_t tile_tokens;  // floor(rows / G)
  int32_t kv_tile;      // keys per inner iteration
};

PS_HD FlatGeom flat_geom(int32_t g, int32_t d) {
  FlatGeom f;
  f.rows = kWaves * kWaveRows;
  f.tile_tokens = g > 0 ? f.rows / g : 0;
  f.kv_tile = d >= 256 ? 32 : 64;
  return f;
}

// Paged: R = draft_len * G rows, split into row blocks of 32; the 4 waves
// are row_blocks x key_streams.  Each wave eats 32 keys per iteration, so
// one iteration of the workgroup loads key_streams * 32 keys.
struct PagedGeom {
  int32_t rows;         // draft_len * G
  int32_t row_blocks;   // ceil(rows / 32) in {1, 2, 4}
  int32_t key_streams;  // 4 / row_blocks
  int32_t kv_tile;      // keys per workgroup iteration = key_streams * 32
};

PS_HD PagedGeom paged_geom(int32_t draft_len, int32_t g, int32_t d, bool f32) {
  PagedGeom p;
  p.rows = draft_len * g;
  int32_t rb = cdiv32(p.rows, kWaveRows);
  p.row_blocks = rb <= 1 ? 1 : (rb <= 2 ? 2 : 4);
  // fp32 K and V tiles of 128 keys x 256 would not fit in LDS: use 64 keys
  if (f32 && d >= 256 && p.row_blocks == 1) p.row_blocks = 2;
  p.key_streams = kWaves / p.row_blocks;
  p.kv_tile = p.key_streams * kWaveRows;
  return p;
}

// Split heuristic: aim at about 512 workgroups (two per CU on a 256-CU part)
// without making a split shorter than one workgroup iteration.  Depends only
// on shapes, so the workspace size is a pure function of the descriptor.
constexpr int32_t kTargetWorkgroups = 512;

struct Splits {
  int32_t n_splits;
  int32_t split_len;
};

PS_HD Splits paged_splits(int32_t batch, int32_t hkv, int32_t max_prefix_len, int32_t kv_tile) {
  Splits s;
  int64_t pairs = (int64_t)batch * hkv;
  if (pairs <= 0 || max_prefix_len <= 0) {
    s.n_splits = 1;
    s.split_len = kv_tile;
    return s;
  }
  int64_t want = cdiv64(kTargetWorkgroups, pairs);
  int64_t max_n = cdiv64(max_prefix_len, kv_tile);
  int64_t n = want < max_n ? want : max_n;
  if (n < 1) n = 1;
  int64_t per = cdiv64(max_prefix_len, n);
  int64_t len = cdiv64(per, kv_tile) * kv_tile;
  s.split_len = (int32_t)len;
  s.n_splits = (int32_t)cdiv64(max_prefix_len, len);
  return s;
}

// ---------------------------------------------------------------- flat plan
PS_HD int64_t flat_items_per_head_ub(int64_t prefix_len, int64_t total, int64_t nseg, int64_t tt) {
  return cdiv64(prefix_len, tt) + (total - prefix_len) / tt + nseg;
}

// Item j of one kv head.  seg_offsets: N+1 entries (may be null when N == 0).
PS_HD Item flat_item(int32_t j, int32_t h_kv, int32_t prefix_len, int32_t nseg,
                     const int32_t* seg_offsets, int32_t tt) {
  Item it{kNone, h_kv, -1, 0, 0, 0, 0, 0, 0, 0};
  int32_t rem = j;
  int32_t a = prefix_len;
  for (int32_t i = 0; i < nseg; ++i) {
    int32_t b = seg_offsets[i + 1];
    int32_t nt = cdiv32(b - a, tt);
    if (rem < nt) {
      int32_t t = nt - 1 - rem;
      it.kind = kFlatSuffix;
      it.seg = i;
      it.q_begin = a + t * tt;
      it.q_end = imin(it.q_begin + tt, b);
      it.r0_begin = 0;
      it.r0_end = prefix_len;
      it.r1_begin = a;
      it.r1_end = it.q_end;
      return it;
    }
    rem -= nt;
    a = b;
  }
  int32_t npre = cdiv32(prefix_len, tt);
  if (rem < npre) {
    int32_t t = npre - 1 - rem;
    it.kind = kFlatPrefix;
    it.q_begin = t * tt;
    it.q_end = imin(it.q_begin + tt, prefix_len);
    it.r0_begin = 0;
    it.r0_end = it.q_end;
  }
  return it;
}

// ---------------------------------------------------------------- paged plan
PS_HD Item paged_item(int32_t blk, int32_t hkv, int32_t n_splits, int32_t split_len,
                      int32_t draft_len, const int32_t* prefix_lens) {
  Item it;
  int32_t s = blk % n_splits;
  int32_t h = (blk / n_splits) % hkv;
  int32_t b = blk / (n_splits * hkv);
  int32_t pl = prefix_lens[b];
  int64_t lo = (int64_t)s * split_len;
  int64_t hi = lo + split_len;
  it.kind = kPagedSplit;
  it.h_kv = h;
  it.seg = b;
  it.q_begin = 0;
  it.q_end = draft_len;
  it.r0_begin = (int32_t)(lo < pl ? lo : pl);
  it.r0_end = (int32_t)(hi < pl ? hi : pl);
  it.r1_begin = 0;
  it.r1_end = 0;
  it.split = s;
  return it;
}

}  // namespace psattn
