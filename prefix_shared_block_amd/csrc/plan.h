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
#include <hip/hip_runtime.h>
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

// Paged.  R = draft_len * G stacked rows.  Three prefix-pass kernels:
//  * register streaming (stream == 2: bf16 / fp8 K/V, R <= 16, power-of-two
//    pages of >= 16 slots): reg_waves(d) waves per workgroup, each streaming
//    its own run of 16-key stages straight into registers several stages
//    ahead (no LDS page table, no barriers), merged in LDS at the end;
//  * wide streaming (stream == 3: bf16 / fp8 K/V, 16 < R <= 64, power-of-two
//    pages of >= 16 slots): four waves per workgroup share 64-key
//    superstages converted to bf16 in LDS, each wave a 32-row x 32-key block
//    of every superstage on 32x32 MFMAs;
//  * LDS streaming (stream == 1: bf16 / fp8 K/V, R <= 64, power-of-two
//    pages of fewer than 16 slots): key stages are
//    copied global -> LDS into a ring of slots, several stages ahead.
//    - R <= 16 with bf16: one-wave workgroups over 16-key stages (3 slots),
//      the wave holding all rows and head-dim columns, no barriers;
//    - otherwise: four-wave workgroups over 32-key stages (ring as deep as
//      128 KiB of LDS allows, at most 8 slots); the waves split the rows into
//      row_groups groups of qblocks 16-row blocks and the head dimension into
//      4 / row_groups slices;
//  * tiled (otherwise): R in 32-row blocks over 4 waves (row_blocks x
//    key_streams), key tiles of key_streams * 32 keys shared through LDS.
struct PagedGeom {
  int32_t rows;         // draft_len * G
  int32_t stream;       // 3: wide, 2: register, 1: LDS streaming; 0: tiled kernel
  int32_t waves;        // waves per workgroup
  int32_t stage_keys;   // streaming: keys per stage (16 or 32)
  int32_t ring;         // streaming: LDS slots
  int32_t max_pages;    // streaming: page-table entries kept in LDS
  int32_t qblocks;      // streaming: 16-row blocks per wave
  int32_t row_groups;   // streaming: row groups (head-dim slices = waves / row_groups)
  int32_t row_blocks;   // tiled: 32-row blocks (1, 2 or 4)
  int32_t key_streams;  // tiled: 4 / row_blocks
  int32_t kv_tile;      // keys consumed by one workgroup iteration
  int32_t wg_per_cu;    // workgroups one CU can hold (LDS-limited estimate)
};

// waves per workgroup of the register-streaming kernel (each wave streams
// its own share of the split; 8 share a CU at two per SIMD up to D = 128)
PS_HD constexpr int32_t reg_waves(int32_t d) { return d <= 128 ? 8 : 4; }

constexpr int32_t kStreamMaxPages = 512;       // four-wave workgroups
constexpr int32_t kStreamMaxPagesSmall = 128;  // one-wave workgroups
constexpr int32_t kLdsPerCu = 160 * 1024;

PS_HD PagedGeom paged_geom(int32_t draft_len, int32_t g, int32_t d, int32_t kv_dtype,
                           int32_t page_size) {
  PagedGeom p;
  p.rows = draft_len * g;
  const int32_t es = kv_dtype == 0 ? 4 : (kv_dtype == 1 ? 2 : 1);
  const bool pow2_pages = page_size > 0 && (page_size & (page_size - 1)) == 0;
  p.stream = (kv_dtype != 0 && p.rows <= 64 && pow2_pages) ? 1 : 0;
  p.row_blocks = 0;
  p.key_streams = 0;
  if (p.stream && p.rows > 16 && page_size >= 16) {
    p.stream = 3;
    p.waves = kWaves;
    p.stage_keys = 64;
    p.ring = 0;
    p.max_pages = 0;
    p.qblocks = 0;
    p.row_groups = 2;
    p.kv_tile = 64;
    p.wg_per_cu = 1;
    return p;
  }
  if (p.stream && p.rows <= 16 && page_size >= 16) {
    p.stream = 2;
    p.waves = reg_waves(d);
    p.stage_keys = 16;
    p.ring = 0;
    p.max_pages = 0;
    p.qblocks = 1;
    p.row_groups = 1;
    p.kv_tile = 16;
    // register-limited residency: 8 waves per CU (16 for D = 64)
    p.wg_per_cu = d <= 64 ? 2 : 1;
    return p;
  }
  if (p.stream) {
    int32_t lds;
    if (kv_dtype == 1 && p.rows <= 16) {
      p.waves = 1;
      p.stage_keys = 16;
      p.ring = 3;
      p.max_pages = kStreamMaxPagesSmall;
      p.qblocks = 1;
      p.row_groups = 1;
      lds = p.ring * 2 * p.stage_keys * d * es + 4 * p.max_pages;
      p.wg_per_cu = kLdsPerCu / lds;
      if (p.wg_per_cu > 8) p.wg_per_cu = 8;
    } else {
      p.waves = kWaves;
      p.stage_keys = 32;
      const int32_t slot = 2 * p.stage_keys * d * es;
      p.ring = 131072 / slot > 8 ? 8 : 131072 / slot;
      p.max_pages = kStreamMaxPages;
      if (p.rows <= 16) {
        p.qblocks = 1;
        p.row_groups = 1;
      } else if (p.rows <= 32) {
        p.qblocks = 1;
        p.row_groups = 2;
      } else if (d >= 256) {  // keep 256-wide rows at one block per wave (register budget)
        p.qblocks = 1;
        p.row_groups = 4;
      } else {
        p.qblocks = 2;
        p.row_groups = 2;
      }
      lds = p.ring * slot + 4 * p.max_pages;
      p.wg_per_cu = kLdsPerCu / lds;
    }
    p.kv_tile = p.stage_keys;
    return p;
  }
  int32_t rb = cdiv32(p.rows, kWaveRows);
  p.waves = kWaves;
  p.stage_keys = 0;
  p.ring = 0;
  p.max_pages = 0;
  p.qblocks = 0;
  p.row_groups = 0;
  p.row_blocks = rb <= 1 ? 1 : (rb <= 2 ? 2 : 4);
  // fp32 K and V tiles of 128 keys x 256 would not fit in LDS: use 64 keys
  if (kv_dtype == 0 && d >= 256 && p.row_blocks == 1) p.row_blocks = 2;
  p.key_streams = kWaves / p.row_blocks;
  p.kv_tile = p.key_streams * kWaveRows;
  p.wg_per_cu = 2;
  return p;
}

// Split heuristic: aim at filling every CU of a 256-CU part with as many
// workgroups as its LDS holds, without making a split shorter than one
// workgroup iteration, without letting the fp32 partial results (R x D x 4
// bytes per split) exceed an eighth of the K/V bytes a split reads, with the
// split's page list fitting in LDS (LDS streaming kernel) and with at most 64
// splits (register and wide streaming kernels).  Depends
// only on shapes, so the workspace size is a pure function of the descriptor.
struct Splits {
  int32_t n_splits;
  int32_t split_len;
};

PS_HD Splits paged_splits(int32_t batch, int32_t hkv, int32_t max_prefix_len, int32_t page_size,
                          int32_t d, int32_t kv_dtype, const PagedGeom& geo) {
  Splits s;
  const int32_t kv_tile = geo.kv_tile;
  int64_t pairs = (int64_t)batch * hkv;
  if (pairs <= 0 || max_prefix_len <= 0) {
    s.n_splits = 1;
    s.split_len = kv_tile;
    return s;
  }
  const int64_t es = kv_dtype == 0 ? 4 : (kv_dtype == 1 ? 2 : 1);
  const int64_t target = 256 * (int64_t)(geo.wg_per_cu > 0 ? geo.wg_per_cu : 1);
  int64_t want = cdiv64(target, pairs);
  // partial bytes per split <= K/V bytes per split / 8
  const int64_t min_len = cdiv64(16 * (int64_t)geo.rows, es);
  const int64_t max_by_partials = max_prefix_len / (min_len > 0 ? min_len : 1);
  if (want > max_by_partials) want = max_by_partials;
  // the merge of the register and wide streaming kernels holds one split
  // weight per lane
  if (geo.stream >= 2 && want > 64) want = 64;
  int64_t max_n = cdiv64(max_prefix_len, kv_tile);
  int64_t n = want < max_n ? want : max_n;
  if (n < 1) n = 1;
  int64_t per = cdiv64(max_prefix_len, n);
  int64_t len = cdiv64(per, kv_tile) * kv_tile;
  if (geo.stream == 1) {
    int64_t cap = ((int64_t)(geo.max_pages - 2) * page_size / kv_tile) * kv_tile;
    if (cap < kv_tile) cap = kv_tile;
    if (len > cap) len = cap;
  }
  s.split_len = (int32_t)len;
  s.n_splits = (int32_t)cdiv64(max_prefix_len, len);
  return s;
}

// ------------------------------------------------- backward (flat) dK/dV plan
// The key-major pass of the backward takes keys [k0, k1) of one kv head (at
// most kBwdKeys, inside the prefix or inside one rollout) against the query
// tokens [r0, r1) of one chunk (at most `rc` tokens) of a row range that sees
// those keys.  Prefix keys are seen by the prefix rows from k0 on and by every
// rollout's rows; a rollout's keys by that rollout's rows from k0 on, and
// (multi-level sharing, seg_parent set) by every row of each segment that
// descends from it.  Items of one kv head, in order: the prefix key tiles,
// each with its prefix-row chunks and then every rollout's chunks (rollouts
// in order); then every rollout's key tiles in order, each with its own row
// chunks and then the chunks of its descendants (in segment order).  A
// descendant follows its ancestors in the buffer, so its rows lie past every
// key of the tile: the tile is wholly visible to them.
constexpr int kBwdKeys = 128;

// Segment `anc` is a proper ancestor of segment s: the walk up s's parents,
// which ends at -1 (the prefix) or at an entry outside [-1, child), the same
// walk as the forward's, meets it.
PS_HD bool seg_has_ancestor(const int32_t* seg_parent, int32_t s, int32_t anc) {
  int32_t child = s;
  int32_t p = seg_parent[s];
  while (p >= 0 && p < child) {
    if (p == anc) return true;
    child = p;
    p = seg_parent[p];
  }
  return false;
}

struct BwdItem {
  int32_t valid, k0, k1, r0, r1;
};

PS_HD BwdItem dkdv_item(int32_t j, int32_t prefix_len, int32_t nseg, const int32_t* seg_offsets,
                        const int32_t* seg_parent, int32_t rc) {
  BwdItem it{0, 0, 0, 0, 0};
  int32_t rem = j;
  int32_t sr = 0;  // chunks of all rollouts' rows
  for (int32_t i = 0; i < nseg; ++i) sr += cdiv32(seg_offsets[i + 1] - seg_offsets[i], rc);
  const int32_t npk = cdiv32(prefix_len, kBwdKeys);
  for (int32_t t = 0; t < npk; ++t) {
    const int32_t k0 = t * kBwdKeys;
    const int32_t np = cdiv32(prefix_len - k0, rc);
    if (rem < np + sr) {
      it.k0 = k0;
      it.k1 = imin(k0 + kBwdKeys, prefix_len);
      if (rem < np) {
        it.valid = 1;
        it.r0 = k0 + rem * rc;
        it.r1 = imin(it.r0 + rc, prefix_len);
        return it;
      }
      rem -= np;
      for (int32_t i = 0; i < nseg; ++i) {
        const int32_t a = seg_offsets[i], b = seg_offsets[i + 1];
        const int32_t ni = cdiv32(b - a, rc);
        if (rem < ni) {
          it.valid = 1;
          it.r0 = a + rem * rc;
          it.r1 = imin(it.r0 + rc, b);
          return it;
        }
        rem -= ni;
      }
      it.k0 = it.k1 = 0;
      return it;
    }
    rem -= np + sr;
  }
  for (int32_t i = 0; i < nseg; ++i) {
    const int32_t a = seg_offsets[i], b = seg_offsets[i + 1];
    for (int32_t k0 = a; k0 < b; k0 += kBwdKeys) {
      const int32_t n = cdiv32(b - k0, rc);
      if (rem < n) {
        it.valid = 1;
        it.k0 = k0;
        it.k1 = imin(k0 + kBwdKeys, b);
        it.r0 = k0 + rem * rc;
        it.r1 = imin(it.r0 + rc, b);
        return it;
      }
      rem -= n;
      if (!seg_parent) continue;
      for (int32_t e = i + 1; e < nseg; ++e) {
        if (!seg_has_ancestor(seg_parent, e, i)) continue;
        const int32_t ae = seg_offsets[e], be = seg_offsets[e + 1];
        const int32_t ne = cdiv32(be - ae, rc);
        if (rem < ne) {
          it.valid = 1;
          it.k0 = k0;
          it.k1 = imin(k0 + kBwdKeys, b);
          it.r0 = ae + rem * rc;
          it.r1 = imin(it.r0 + rc, be);
          return it;
        }
        rem -= ne;
      }
    }
  }
  return it;
}

// Upper bound on the dK/dV items of one kv head from host scalars only
// (chain: multi-level sharing, where a rollout key tile also takes the
// chunks of its descendants, at most all rollouts' chunks).
PS_HD int64_t dkdv_items_per_head_ub(int64_t prefix_len, int64_t total, int64_t nseg, int64_t max_seg,
                                     int64_t rc, bool chain) {
  const int64_t suf = total - prefix_len;
  const int64_t sr = cdiv64(suf, rc) + nseg;  // >= sum_i ceil(S_i / rc)
  const int64_t pre = cdiv64(prefix_len, kBwdKeys) * (cdiv64(prefix_len, rc) + sr);
  const int64_t rtiles = suf / kBwdKeys + nseg;  // >= number of rollout key tiles
  return pre + rtiles * (cdiv64(max_seg, rc) + (chain ? sr : 0));
}

// Ragged draft lengths: request b's draft rows (of q, o, lse, k_ext, v_ext)
// are qo_indptr[b] .. qo_indptr[b+1]; without qo_indptr every request has
// draft_len rows at b * draft_len.
PS_HD int32_t draft_base(const int32_t* qo_indptr, int32_t b, int32_t draft_len) {
  return qo_indptr ? qo_indptr[b] : b * draft_len;
}
PS_HD int32_t draft_count(const int32_t* qo_indptr, int32_t b, int32_t draft_len) {
  return qo_indptr ? qo_indptr[b + 1] - qo_indptr[b] : draft_len;
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
