// launch.h -- internal interface between the C-ABI host code and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace psattn {

struct FlatArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seg_offsets;
  int32_t prefix_len;
  int32_t nseg;
  int32_t hq;
  int32_t hkv;
  int32_t g;
  int32_t tile_tokens;
  float scale_log2;  // sm_scale * log2(e)
  const int32_t* seg_parent;  // [N] parent segment (-1: the prefix), or null: one level
};

struct PagedArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const void* k_ext;
  const void* v_ext;
  void* o;
  float* lse;
  const int32_t* prefix_lens;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  float* part_o;    // [B, Hkv, n_splits, R, D]  normalised partial outputs (fp32, or bf16 with part_bf16)
  float* part_lse;  // [B, Hkv, n_splits, R]     log2-domain partial LSE
  int32_t part_bf16;  // 1: part_o holds bf16 (the register and wide split passes and their merge)
  int32_t batch;
  int32_t draft_len;
  int32_t page_size;
  int32_t hq;
  int32_t hkv;
  int32_t g;
  int32_t rows;  // draft_len * g
  int32_t n_splits;
  int32_t split_len;
  float scale_log2;  // sm_scale * k_scale * log2(e)
  float v_scale;
  const uint8_t* draft_mask;  // [B, L, L] draft visibility (nonzero: visible), or null: causal
  const int32_t* qo_indptr;   // [B + 1] ragged draft rows, or null: draft_len rows per request
};

// Backward of the flat forward (bf16).  Workspace: lse2 and delta [T, Hq]
// fp32, acc_k and acc_v [T, Hkv, D] fp32, the dK/dV item table.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;   // forward LSE, natural log, [T, Hq]
  const void* dout;   // dO [T, Hq, D]
  void* dq;
  void* dk;
  void* dv;
  float* lse2;   // LSE log2(e)
  float* delta;  // sum_d dO O
  float* acc_k;
  float* acc_v;
  int32_t* item_tab;  // [n_tab + 1][4] dK/dV items of one kv head: k0, k1, r0, r1 (k1 <= k0: none); entry n_tab: the first item past the table
  int32_t n_tab;
  const int32_t* seg_offsets;
  const int32_t* seg_parent;  // [N] parent segment (-1: the prefix), or null: one level
  int64_t total_tokens;
  int32_t prefix_len;
  int32_t nseg;
  int32_t hq;
  int32_t hkv;
  int32_t g;
  int32_t tile_tokens;  // query tokens per dQ item (the forward's)
  int32_t row_chunk;    // query tokens per dK/dV item
  float scale_log2;     // sm_scale * log2(e)
  float sm_scale;
};
// pre (delta, lse2, zeroed accumulators, the item table), dQ, dK/dV and the
// final conversion, defined in psattn_bwd.hip
int launch_flat_bwd(const BwdArgs& a, int d, int64_t dq_blocks, int64_t dkdv_blocks, void* stream);

// dtype codes follow psattn_dtype (0 f32, 1 bf16, 2 fp8 e4m3fn)
int launch_flat(const FlatArgs& a, int d, int dtype, int64_t n_blocks, void* stream);
// bf16 flat kernel, defined in psattn_flat.hip
int launch_flat_bf16(const FlatArgs& a, int d, int64_t n_blocks, void* stream);
struct PagedGeom;
int launch_paged(const PagedArgs& a, int d, int q_dtype, int kv_dtype, const PagedGeom& geo,
                 int64_t n_blocks, void* stream);
// streaming prefix pass (bf16 / fp8 K/V), defined in psattn_stream.hip
int launch_paged_stream(const PagedArgs& a, int d, int kv_dtype, const PagedGeom& geo, int64_t n_blocks,
                        void* stream);
// register-streamed prefix pass with the draft block folded into each
// request's last split (bf16 / fp8 K/V, R <= 16), and the matching merge of
// the splits (no draft work), defined in psattn_regstream.hip
int launch_paged_reg(const PagedArgs& a, int d, int kv_dtype, int64_t n_blocks, void* stream);
int launch_paged_merge(const PagedArgs& a, int d, int q_dtype, void* stream);
// wide prefix pass (bf16 / fp8 K/V, 16 < R <= 64) with the draft block folded
// into each request's last split, defined in psattn_widestream.hip
int launch_paged_wide(const PagedArgs& a, int d, int kv_dtype, int64_t n_blocks, void* stream);
// log-sum-exp combine + draft block, defined in psattn_kernels.hip
int launch_paged_combine(const PagedArgs& a, int d, int q_dtype, int kv_dtype, void* stream);
int launch_plan_dump(int mode, const FlatArgs* fa, const PagedArgs* pa, int64_t n_items,
                     int32_t* items, void* stream);
const char* hip_error_string(int err);
// device address of the allocation-free scratch array
// (PSATTN_NOALLOC_SCRATCH_BYTES) on the device of `stream`, defined in
// psattn_noalloc.hip
int noalloc_scratch(void* stream, void** ptr);

}  // namespace psattn
