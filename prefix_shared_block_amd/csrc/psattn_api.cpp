// psattn_api.cpp -- C-ABI entry points: host-side validation, planning of the
// launch geometry, and dispatch to the gfx950 kernels.  Validation runs to
// completion before the first HIP call, so an error status leaves every
// output untouched and enqueues nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/psattn.h"
#include "launch.h"
#include "mla.h"
#include "plan.h"

using namespace psattn;

namespace {

thread_local std::string g_last_error;

psattn_status fail(psattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Everything a launch needs, derived from the descriptor on the host only.
struct Plan {
  int mode = 0;
  int32_t g = 0;
  // flat
  FlatGeom fg{};
  int64_t flat_blocks = 0;
  // paged
  PagedGeom pg{};
  Splits sp{};
  int64_t paged_blocks = 0;
  size_t ws_bytes = 0;
  size_t ws_lse_offset = 0;
};

constexpr size_t kWsAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Host-scalar validation of the descriptor and the shape/dtype arguments.
psattn_status check_common(const psattn_desc* d, int32_t hq, int32_t hkv, int32_t hd,
                           psattn_dtype q_dt, psattn_dtype kv_dt, Plan* plan) {
  if (!d) return fail(PSATTN_E_INVAL, "desc is NULL");
  if (d->mode != PSATTN_MODE_FLAT && d->mode != PSATTN_MODE_PAGED)
    return fail(PSATTN_E_INVAL, "mode %d is neither flat (0) nor paged (1)", d->mode);
  if (hq <= 0 || hkv <= 0) return fail(PSATTN_E_INVAL, "head counts must be positive (hq=%d hkv=%d)", hq, hkv);
  if (hq % hkv != 0) return fail(PSATTN_E_INVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  if (hd != 64 && hd != 128 && hd != 256)
    return fail(PSATTN_E_UNSUPPORTED, "head dim %d not in {64, 128, 256}", hd);
  const bool f32pair = q_dt == PSATTN_F32 && kv_dt == PSATTN_F32;
  const bool bfpair = q_dt == PSATTN_BF16 && kv_dt == PSATTN_BF16;
  const bool fp8pair = q_dt == PSATTN_BF16 && kv_dt == PSATTN_FP8_E4M3;
  if ((int)q_dt < 0 || (int)q_dt > 2 || (int)kv_dt < 0 || (int)kv_dt > 2)
    return fail(PSATTN_E_INVAL, "unknown dtype code (q=%d kv=%d)", (int)q_dt, (int)kv_dt);
  if (!(f32pair || bfpair || (fp8pair && d->mode == PSATTN_MODE_PAGED)))
    return fail(PSATTN_E_UNSUPPORTED, "dtype pair (q=%d, kv=%d) not supported in mode %d", (int)q_dt,
                (int)kv_dt, d->mode);
  plan->mode = d->mode;
  plan->g = hq / hkv;

  if (d->mode == PSATTN_MODE_FLAT) {
    const int64_t t = d->total_tokens;
    if (t < 0 || t > INT32_MAX) return fail(PSATTN_E_INVAL, "total_tokens %lld out of range", (long long)t);
    if (d->prefix_len < 0 || d->prefix_len > t)
      return fail(PSATTN_E_INVAL, "prefix_len %d outside [0, total_tokens=%lld]", d->prefix_len, (long long)t);
    if (d->num_segments < 0) return fail(PSATTN_E_INVAL, "num_segments %d < 0", d->num_segments);
    if (d->num_segments == 0 && t != d->prefix_len)
      return fail(PSATTN_E_INVAL, "num_segments = 0 requires total_tokens == prefix_len");
    if (d->num_segments > 0 && !d->seg_offsets) return fail(PSATTN_E_INVAL, "seg_offsets is NULL");
    if (d->max_seg_len < 0) return fail(PSATTN_E_INVAL, "max_seg_len %d < 0", d->max_seg_len);
    if ((int64_t)d->num_segments * d->max_seg_len < t - d->prefix_len)
      return fail(PSATTN_E_INVAL, "num_segments * max_seg_len < total_tokens - prefix_len");
    if (plan->g > kWaves * kWaveRows)
      return fail(PSATTN_E_UNSUPPORTED, "GQA group %d exceeds %d stacked rows", plan->g, kWaves * kWaveRows);
    if (d->seg_parent && !bfpair)
      return fail(PSATTN_E_UNSUPPORTED, "seg_parent (multi-level sharing) takes bf16 only");
    plan->fg = flat_geom(plan->g, hd);
    const int64_t per_head =
        t == 0 ? 0 : flat_items_per_head_ub(d->prefix_len, t, d->num_segments, plan->fg.tile_tokens);
    plan->flat_blocks = per_head * hkv;
    if (plan->flat_blocks > INT32_MAX) return fail(PSATTN_E_UNSUPPORTED, "grid too large");
    plan->ws_bytes = 0;
  } else {
    if (d->batch < 0) return fail(PSATTN_E_INVAL, "batch %d < 0", d->batch);
    if (d->draft_len < 1) return fail(PSATTN_E_INVAL, "draft_len %d < 1", d->draft_len);
    if (d->page_size < 1) return fail(PSATTN_E_INVAL, "page_size %d < 1", d->page_size);
    if (d->num_pages < 0) return fail(PSATTN_E_INVAL, "num_pages %d < 0", d->num_pages);
    if (d->max_prefix_len < 0) return fail(PSATTN_E_INVAL, "max_prefix_len %d < 0", d->max_prefix_len);
    if ((int64_t)d->max_prefix_len > (int64_t)d->num_pages * d->page_size)
      return fail(PSATTN_E_INVAL, "max_prefix_len exceeds the pool (num_pages * page_size)");
    if (d->batch > 0 && (!d->prefix_lens || !d->kv_indptr || !d->kv_indices))
      return fail(PSATTN_E_INVAL, "prefix_lens / kv_indptr / kv_indices must not be NULL");
    if (d->batch > 0 && (!d->k_ext || !d->v_ext)) return fail(PSATTN_E_INVAL, "k_ext / v_ext must not be NULL");
    const int64_t rows = (int64_t)d->draft_len * plan->g;
    if (rows > kWaves * kWaveRows)
      return fail(PSATTN_E_UNSUPPORTED, "draft_len * G = %lld exceeds %d stacked rows", (long long)rows,
                  kWaves * kWaveRows);
    if ((int64_t)d->batch * d->draft_len > INT32_MAX / 2) return fail(PSATTN_E_UNSUPPORTED, "batch too large");
    plan->pg = paged_geom(d->draft_len, plan->g, hd, (int32_t)kv_dt, d->page_size);
    plan->sp = paged_splits(d->batch, hkv, d->max_prefix_len, d->page_size, hd, (int32_t)kv_dt, plan->pg);
    plan->paged_blocks = (int64_t)d->batch * hkv * plan->sp.n_splits;
    if (plan->paged_blocks > INT32_MAX) return fail(PSATTN_E_UNSUPPORTED, "grid too large");
    const size_t prow = (size_t)d->batch * hkv * plan->sp.n_splits * plan->pg.rows;
    // the register and wide split passes (stream 2, 3) keep their partial O
    // in bf16 (half the bytes written and read back by the merge), the
    // others in fp32
    const size_t pes = (plan->pg.stream == 2 || plan->pg.stream == 3) ? 2 : 4;
    const size_t o_bytes = round_up(prow * hd * pes, kWsAlign);
    plan->ws_lse_offset = o_bytes;
    plan->ws_bytes = d->batch == 0 ? 0 : o_bytes + round_up(prow * sizeof(float), kWsAlign);
  }
  return PSATTN_OK;
}

// Everything psattn_fwd checks apart from the workspace; *empty: nothing to
// enqueue (a valid call with no rows).
psattn_status check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                        psattn_dtype q_dtype, psattn_dtype kv_dtype, float k_scale, float v_scale, Plan* p,
                        bool* empty) {
  psattn_status st = check_common(desc, hq, hkv, d, q_dtype, kv_dtype, p);
  if (st != PSATTN_OK) return st;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(PSATTN_E_INVAL, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (!(k_scale > 0.f) || !std::isfinite(k_scale) || !(v_scale > 0.f) || !std::isfinite(v_scale))
    return fail(PSATTN_E_INVAL, "k_scale / v_scale must be finite and > 0");
  *empty = desc->mode == PSATTN_MODE_FLAT ? desc->total_tokens == 0 : desc->batch == 0;
  if (*empty) return PSATTN_OK;
  if (!q || !k || !v || !o || !lse) return fail(PSATTN_E_INVAL, "q, k, v, o and lse must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(PSATTN_E_INVAL, "q/k/v/o must be 16-byte aligned and lse 4-byte aligned");
  if (desc->mode == PSATTN_MODE_PAGED && (!aligned(desc->k_ext, 4) || !aligned(desc->v_ext, 4)))
    return fail(PSATTN_E_INVAL, "k_ext / v_ext misaligned");
  if (desc->mode == PSATTN_MODE_FLAT && (k_scale != 1.0f || v_scale != 1.0f))
    return fail(PSATTN_E_UNSUPPORTED, "k_scale / v_scale must be 1 in flat mode");
  return PSATTN_OK;
}

// ---------------------------------------------------------------- backward
constexpr int32_t kBwdRowChunk = 512;  // query tokens per dK/dV item

struct BwdPlan {
  Plan base;
  int64_t dq_blocks = 0;
  int64_t dkdv_blocks = 0;
  size_t off_delta = 0, off_acck = 0, off_accv = 0, off_items = 0, ws_bytes = 0;
  int64_t n_tab = 0;  // dK/dV items of one kv head in the one-item launch (its table's entries)
};

psattn_status check_bwd(const psattn_desc* d, int32_t hq, int32_t hkv, int32_t hd, psattn_dtype dt,
                        BwdPlan* bp) {
  if (d && d->mode != PSATTN_MODE_FLAT) return fail(PSATTN_E_UNSUPPORTED, "the backward covers the flat layout only");
  psattn_status st = check_common(d, hq, hkv, hd, dt, dt, &bp->base);
  if (st != PSATTN_OK) return st;
  if (dt != PSATTN_BF16) return fail(PSATTN_E_UNSUPPORTED, "the backward takes bf16 only");
  if (hd != 64 && hd != 128 && hd != 256)
    return fail(PSATTN_E_UNSUPPORTED, "the backward takes head dims 64, 128 and 256 (got %d)", hd);
  if (bp->base.g > 64) return fail(PSATTN_E_UNSUPPORTED, "the backward takes GQA groups up to 64 (got %d)", bp->base.g);
  const int64_t t = d->total_tokens;
  bp->dq_blocks = bp->base.flat_blocks;
  bp->n_tab = t == 0 ? 0
                     : dkdv_items_per_head_ub(d->prefix_len, t, d->num_segments, d->max_seg_len, kBwdRowChunk,
                                              d->num_segments > 0 && d->seg_parent != nullptr);
  bp->dkdv_blocks = bp->n_tab * hkv;
  if (bp->dkdv_blocks > INT32_MAX) return fail(PSATTN_E_UNSUPPORTED, "grid too large");
  const size_t rows = (size_t)t * hq * sizeof(float);
  const size_t acc = (size_t)t * hkv * hd * sizeof(float);
  bp->off_delta = round_up(rows, kWsAlign);
  bp->off_acck = bp->off_delta + round_up(rows, kWsAlign);
  bp->off_accv = bp->off_acck + round_up(acc, kWsAlign);
  bp->off_items = bp->off_accv + round_up(acc, kWsAlign);
  // the table's n_tab entries, then one for the first item past them (which
  // tells the walking launch whether it has any work)
  bp->ws_bytes = t == 0 ? 0 : bp->off_items + round_up((size_t)(bp->n_tab + 1) * 4 * sizeof(int32_t), kWsAlign);
  return PSATTN_OK;
}

void fill_info(const Plan& p, psattn_plan_info* info) {
  if (!info) return;
  std::memset(info, 0, sizeof(*info));
  if (p.mode == PSATTN_MODE_FLAT) {
    info->n_items = p.flat_blocks;
    info->tile_tokens = p.fg.tile_tokens;
    info->rows_per_tile = p.fg.rows;
    info->kv_tile = p.fg.kv_tile;
  } else {
    info->n_items = p.paged_blocks;
    info->rows_per_tile = p.pg.rows;
    info->n_splits = p.sp.n_splits;
    info->split_len = p.sp.split_len;
    info->kv_tile = p.pg.kv_tile;
  }
}

}  // namespace

extern "C" {

const char* psattn_status_string(psattn_status st) {
  switch (st) {
    case PSATTN_OK: return "ok";
    case PSATTN_E_INVAL: return "invalid argument";
    case PSATTN_E_UNSUPPORTED: return "unsupported configuration";
    case PSATTN_E_WORKSPACE: return "workspace missing or too small";
    case PSATTN_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* psattn_last_error(void) { return g_last_error.c_str(); }

size_t psattn_workspace_size(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                             psattn_dtype q_dtype, psattn_dtype kv_dtype) {
  Plan p;
  if (check_common(desc, hq, hkv, d, q_dtype, kv_dtype, &p) != PSATTN_OK) return 0;
  return p.ws_bytes;
}

psattn_status psattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                         psattn_dtype q_dtype, psattn_dtype kv_dtype, float k_scale, float v_scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Plan p;
  bool empty = false;
  psattn_status st = check_fwd(q, k, v, o, lse, desc, hq, hkv, d, sm_scale, q_dtype, kv_dtype, k_scale, v_scale,
                               &p, &empty);
  if (st != PSATTN_OK || empty) return st;
  if (p.ws_bytes > 0) {
    if (!workspace || workspace_bytes < p.ws_bytes)
      return fail(PSATTN_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, kWsAlign)) return fail(PSATTN_E_INVAL, "workspace must be 256-byte aligned");
  }
  const float log2e = 1.4426950408889634f;
  int err = 0;
  if (desc->mode == PSATTN_MODE_FLAT) {
    FlatArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.seg_offsets = desc->seg_offsets;
    a.seg_parent = desc->num_segments > 0 ? desc->seg_parent : nullptr;
    a.prefix_len = desc->prefix_len;
    a.nseg = desc->num_segments;
    a.hq = hq;
    a.hkv = hkv;
    a.g = p.g;
    a.tile_tokens = p.fg.tile_tokens;
    a.scale_log2 = sm_scale * log2e;
    err = launch_flat(a, d, (int)q_dtype, p.flat_blocks, stream);
  } else {
    PagedArgs a{};
    a.q = q;
    a.k_pool = k;
    a.v_pool = v;
    a.k_ext = desc->k_ext;
    a.v_ext = desc->v_ext;
    a.o = o;
    a.lse = lse;
    a.prefix_lens = desc->prefix_lens;
    a.kv_indptr = desc->kv_indptr;
    a.kv_indices = desc->kv_indices;
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + p.ws_lse_offset);
    a.part_bf16 = (p.pg.stream == 2 || p.pg.stream == 3) ? 1 : 0;
    a.batch = desc->batch;
    a.draft_len = desc->draft_len;
    a.page_size = desc->page_size;
    a.hq = hq;
    a.hkv = hkv;
    a.g = p.g;
    a.rows = p.pg.rows;
    a.n_splits = p.sp.n_splits;
    a.split_len = p.sp.split_len;
    a.scale_log2 = sm_scale * k_scale * log2e;
    a.v_scale = v_scale;
    a.draft_mask = desc->draft_mask;
    a.qo_indptr = desc->qo_indptr;
    err = launch_paged(a, d, (int)q_dtype, (int)kv_dtype, p.pg, p.paged_blocks, stream);
  }
  if (err) return fail(PSATTN_E_HIP, "kernel launch failed: %s", hip_error_string(err));
  return PSATTN_OK;
}

psattn_status psattn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                                 psattn_dtype q_dtype, psattn_dtype kv_dtype, float k_scale, float v_scale,
                                 void* stream) {
  g_last_error.clear();
  Plan p;
  bool empty = false;
  psattn_status st = check_fwd(q, k, v, o, lse, desc, hq, hkv, d, sm_scale, q_dtype, kv_dtype, k_scale, v_scale,
                               &p, &empty);
  if (st != PSATTN_OK || empty) return st;
  if (p.ws_bytes > PSATTN_NOALLOC_SCRATCH_BYTES)
    return fail(PSATTN_E_UNSUPPORTED,
                "the split scratch of %zu bytes exceeds the %zu bytes the allocation-free entry point holds "
                "(use psattn_fwd with a workspace)",
                p.ws_bytes, (size_t)PSATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (p.ws_bytes > 0) {
    const int err = noalloc_scratch(stream, &ws);
    if (err) return fail(PSATTN_E_HIP, "scratch lookup failed: %s", hip_error_string(err));
    ws_bytes = PSATTN_NOALLOC_SCRATCH_BYTES;
  }
  return psattn_fwd(q, k, v, o, lse, desc, hq, hkv, d, sm_scale, q_dtype, kv_dtype, k_scale, v_scale, ws,
                    ws_bytes, stream);
}

size_t psattn_bwd_workspace_size(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                                 psattn_dtype dtype) {
  g_last_error.clear();
  BwdPlan bp;
  if (check_bwd(desc, hq, hkv, d, dtype, &bp) != PSATTN_OK) return 0;
  return bp.ws_bytes;
}

psattn_status psattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, const psattn_desc* desc,
                         int32_t hq, int32_t hkv, int32_t d, float sm_scale, psattn_dtype dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  BwdPlan bp;
  psattn_status st = check_bwd(desc, hq, hkv, d, dtype, &bp);
  if (st != PSATTN_OK) return st;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(PSATTN_E_INVAL, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (desc->total_tokens == 0) return PSATTN_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(PSATTN_E_INVAL, "q, k, v, o, lse, dout, dq, dk and dv must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return fail(PSATTN_E_INVAL, "tensors must be 16-byte aligned and lse 4-byte aligned");
  if (!workspace || workspace_bytes < bp.ws_bytes)
    return fail(PSATTN_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", bp.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, kWsAlign)) return fail(PSATTN_E_INVAL, "workspace must be 256-byte aligned");
  char* ws = reinterpret_cast<char*>(workspace);
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.lse2 = reinterpret_cast<float*>(ws);
  a.delta = reinterpret_cast<float*>(ws + bp.off_delta);
  a.acc_k = reinterpret_cast<float*>(ws + bp.off_acck);
  a.acc_v = reinterpret_cast<float*>(ws + bp.off_accv);
  a.item_tab = reinterpret_cast<int32_t*>(ws + bp.off_items);
  a.n_tab = (int32_t)bp.n_tab;
  a.seg_offsets = desc->seg_offsets;
  a.seg_parent = desc->num_segments > 0 ? desc->seg_parent : nullptr;
  a.total_tokens = desc->total_tokens;
  a.prefix_len = desc->prefix_len;
  a.nseg = desc->num_segments;
  a.hq = hq;
  a.hkv = hkv;
  a.g = bp.base.g;
  a.tile_tokens = bp.base.fg.tile_tokens;
  a.row_chunk = kBwdRowChunk;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.sm_scale = sm_scale;
  const int err = launch_flat_bwd(a, d, bp.dq_blocks, bp.dkdv_blocks, stream);
  if (err) return fail(PSATTN_E_HIP, "kernel launch failed: %s", hip_error_string(err));
  return PSATTN_OK;
}

psattn_status psattn_mla_fwd(const void* q, const void* ckv, const int32_t* indices, const float* sink, void* o,
                             float* lse, int64_t num_tokens, int32_t num_heads, int32_t dim, int64_t num_kv,
                             int32_t kv_stride, int32_t topk, float sm_scale, psattn_dtype dtype, void* stream) {
  g_last_error.clear();
  if ((int)dtype < 0 || (int)dtype > 2) return fail(PSATTN_E_INVAL, "unknown dtype code %d", (int)dtype);
  if (dtype != PSATTN_BF16) return fail(PSATTN_E_UNSUPPORTED, "the sparse MLA forward takes bf16 only");
  if (dim != kMlaDim) return fail(PSATTN_E_UNSUPPORTED, "latent width %d is not %d", dim, kMlaDim);
  if (num_heads != 32 && num_heads != 64 && num_heads != 128)
    return fail(PSATTN_E_UNSUPPORTED, "num_heads %d not in {32, 64, 128}", num_heads);
  if (num_tokens < 0 || num_tokens > INT32_MAX)
    return fail(PSATTN_E_INVAL, "num_tokens %lld out of range", (long long)num_tokens);
  if (num_kv < 0 || num_kv > INT32_MAX) return fail(PSATTN_E_INVAL, "num_kv %lld out of range", (long long)num_kv);
  if (topk < 0) return fail(PSATTN_E_INVAL, "topk %d < 0", topk);
  if (topk > kMlaMaxTopk) return fail(PSATTN_E_UNSUPPORTED, "topk %d exceeds %d", topk, kMlaMaxTopk);
  if (kv_stride < dim || kv_stride % 8 != 0)
    return fail(PSATTN_E_INVAL, "kv_stride %d must be >= %d and a multiple of 8", kv_stride, dim);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(PSATTN_E_INVAL, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (num_tokens == 0) return PSATTN_OK;
  if (!q || !o || !lse) return fail(PSATTN_E_INVAL, "q, o and lse must not be NULL");
  if (topk > 0 && !indices) return fail(PSATTN_E_INVAL, "indices must not be NULL");
  if (num_kv > 0 && !ckv) return fail(PSATTN_E_INVAL, "ckv must not be NULL");
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(ckv, 16) || !aligned(lse, 4) || !aligned(indices, 4) ||
      !aligned(sink, 4))
    return fail(PSATTN_E_INVAL, "q, o and ckv must be 16-byte aligned; lse, indices and sink 4-byte aligned");
  MlaArgs a{};
  a.q = q;
  a.ckv = ckv;
  a.indices = indices;
  a.sink = sink;
  a.o = o;
  a.lse = lse;
  a.num_tokens = (int32_t)num_tokens;
  a.num_heads = num_heads;
  a.num_kv = (int32_t)num_kv;
  a.kv_stride = kv_stride;
  a.topk = topk;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  const int err = launch_mla(a, false, stream);
  if (err) return fail(PSATTN_E_HIP, "kernel launch failed: %s", hip_error_string(err));
  return PSATTN_OK;
}

psattn_status psattn_mla_dense_fwd(const void* q, const void* ckv, const float* sink, void* o, float* lse,
                                   int64_t num_tokens, int32_t num_heads, int32_t dim, int64_t num_kv,
                                   int32_t kv_stride, float sm_scale, psattn_dtype dtype, void* stream) {
  g_last_error.clear();
  if ((int)dtype < 0 || (int)dtype > 2) return fail(PSATTN_E_INVAL, "unknown dtype code %d", (int)dtype);
  if (dtype != PSATTN_BF16) return fail(PSATTN_E_UNSUPPORTED, "the MLA forward takes bf16 only");
  if (dim != kMlaDim) return fail(PSATTN_E_UNSUPPORTED, "latent width %d is not %d", dim, kMlaDim);
  if (num_heads != 32 && num_heads != 64 && num_heads != 128)
    return fail(PSATTN_E_UNSUPPORTED, "num_heads %d not in {32, 64, 128}", num_heads);
  if (num_tokens < 0 || num_tokens > INT32_MAX)
    return fail(PSATTN_E_INVAL, "num_tokens %lld out of range", (long long)num_tokens);
  if (num_kv < 0 || num_kv > INT32_MAX) return fail(PSATTN_E_INVAL, "num_kv %lld out of range", (long long)num_kv);
  if (num_kv < num_tokens)
    return fail(PSATTN_E_INVAL, "num_kv %lld < num_tokens %lld: the cache must hold the query tokens",
                (long long)num_kv, (long long)num_tokens);
  if (kv_stride < dim || kv_stride % 8 != 0)
    return fail(PSATTN_E_INVAL, "kv_stride %d must be >= %d and a multiple of 8", kv_stride, dim);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(PSATTN_E_INVAL, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
  if (num_tokens == 0) return PSATTN_OK;
  if (!q || !o || !lse || !ckv) return fail(PSATTN_E_INVAL, "q, ckv, o and lse must not be NULL");
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(ckv, 16) || !aligned(lse, 4) || !aligned(sink, 4))
    return fail(PSATTN_E_INVAL, "q, o and ckv must be 16-byte aligned; lse and sink 4-byte aligned");
  MlaArgs a{};
  a.q = q;
  a.ckv = ckv;
  a.indices = nullptr;
  a.sink = sink;
  a.o = o;
  a.lse = lse;
  a.num_tokens = (int32_t)num_tokens;
  a.num_heads = num_heads;
  a.num_kv = (int32_t)num_kv;
  a.kv_stride = kv_stride;
  a.topk = 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  const int err = launch_mla(a, true, stream);
  if (err) return fail(PSATTN_E_HIP, "kernel launch failed: %s", hip_error_string(err));
  return PSATTN_OK;
}

psattn_status psattn_plan_dump(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                               psattn_dtype q_dtype, psattn_dtype kv_dtype, int32_t* items_dev,
                               int64_t capacity, psattn_plan_info* info_host, void* stream) {
  g_last_error.clear();
  Plan p;
  psattn_status st = check_common(desc, hq, hkv, d, q_dtype, kv_dtype, &p);
  if (st != PSATTN_OK) return st;
  fill_info(p, info_host);
  if (!items_dev) return PSATTN_OK;
  const int64_t n = p.mode == PSATTN_MODE_FLAT ? p.flat_blocks : p.paged_blocks;
  if (capacity < n) return fail(PSATTN_E_INVAL, "capacity %lld < %lld items", (long long)capacity, (long long)n);
  FlatArgs fa{};
  PagedArgs pa{};
  fa.seg_offsets = desc->seg_offsets;
  fa.prefix_len = desc->prefix_len;
  fa.nseg = desc->num_segments;
  fa.hkv = hkv;
  fa.tile_tokens = p.fg.tile_tokens;
  pa.prefix_lens = desc->prefix_lens;
  pa.hkv = hkv;
  pa.n_splits = p.sp.n_splits;
  pa.split_len = p.sp.split_len;
  pa.draft_len = desc->draft_len;
  int err = launch_plan_dump(p.mode, &fa, &pa, n, items_dev, stream);
  if (err) return fail(PSATTN_E_HIP, "plan dump launch failed: %s", hip_error_string(err));
  return PSATTN_OK;
}

psattn_status psattn_plan_host(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                               psattn_dtype q_dtype, psattn_dtype kv_dtype, int32_t* items_host,
                               int64_t capacity, psattn_plan_info* info_host) {
  g_last_error.clear();
  Plan p;
  psattn_status st = check_common(desc, hq, hkv, d, q_dtype, kv_dtype, &p);
  if (st != PSATTN_OK) return st;
  fill_info(p, info_host);
  if (!items_host) return PSATTN_OK;
  const int64_t n = p.mode == PSATTN_MODE_FLAT ? p.flat_blocks : p.paged_blocks;
  if (capacity < n) return fail(PSATTN_E_INVAL, "capacity %lld < %lld items", (long long)capacity, (long long)n);
  for (int64_t i = 0; i < n; ++i) {
    Item it;
    if (p.mode == PSATTN_MODE_FLAT)
      it = flat_item((int32_t)(i / hkv), (int32_t)(i % hkv), desc->prefix_len, desc->num_segments,
                     desc->seg_offsets, p.fg.tile_tokens);
    else
      it = paged_item((int32_t)i, hkv, p.sp.n_splits, p.sp.split_len, desc->draft_len, desc->prefix_lens);
    int32_t* o = items_host + i * PSATTN_ITEM_FIELDS;
    o[0] = it.kind;
    o[1] = it.h_kv;
    o[2] = it.seg;
    o[3] = it.q_begin;
    o[4] = it.q_end;
    o[5] = it.r0_begin;
    o[6] = it.r0_end;
    o[7] = it.r1_begin;
    o[8] = it.r1_end;
    o[9] = it.split;
  }
  return PSATTN_OK;
}

}  // extern "C"
