/*
 * psattn.h -- prefix-shared attention forward for AMD gfx950 (MI355X).
 *
 * C ABI of libpsattn.so.  Plain pointers and sizes only.  Unless stated
 * otherwise a pointer is a DEVICE pointer; the library never frees, keeps or
 * allocates caller memory.
 *
 * What is computed.  PrefixSharing PR #50 ("设计简介", design summary) packs
 * a shared prompt P and N rollout suffixes flat as [P | S1 | ... | SN], keeps
 * the prefix K/V once, and controls visibility with a block-causal mask
 * instead of copying the prefix into every rollout (the build_kv route); the
 * result is stated to be exactly that of ordinary causal attention over each
 * expanded sequence [P | Si].  Row r of the packed buffer sees key c iff
 * c <= r and (c < P or c lies in r's own segment).  sglang PR #27382
 * ("实现拆解", implementation breakdown) applies the same idea to EAGLE
 * target-verify: a few draft rows per request read the request's long paged
 * prefix in splits (one partial O and log-sum-exp per split), and a second
 * stage merges the splits by log-sum-exp together with the small causal
 * draft-by-draft block.
 *
 * For every query row r and query head h (kv head g = h / (Hq / Hkv)):
 *     z_c  = sm_scale * <q[r,h,:], K[c,g,:]>      over the keys c that r sees
 *     lse  = ln sum_c exp(z_c)                     (natural log, fp32)
 *     o    = sum_c exp(z_c - lse) * V[c,g,:]       (stored in q's dtype)
 * with K, V multiplied by k_scale, v_scale in paged mode.
 *
 * Execution.  All work is enqueued asynchronously on the caller's stream
 * (a hipStream_t passed as void*, NULL = the null stream).  Nothing is read
 * back from the device: every size the launch needs comes in as a host
 * scalar.  All arguments are validated on the host before the first launch,
 * so an error status means nothing was enqueued and no output was touched.
 * Faults inside kernels (for example a device array that breaks the
 * documented invariants) surface as HIP errors at the caller's next
 * synchronisation.  The library keeps no mutable global state apart from a
 * per-thread last-error string.
 */
#ifndef PSATTN_H_
#define PSATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element storage types. */
typedef enum {
  PSATTN_F32 = 0,       /* IEEE binary32 */
  PSATTN_BF16 = 1,      /* bfloat16 */
  PSATTN_FP8_E4M3 = 2   /* OCP fp8 e4m3fn (bias 7, no inf, max 448) */
} psattn_dtype;

typedef enum {
  PSATTN_OK = 0,
  PSATTN_E_INVAL = 1,        /* malformed argument (null, negative, misaligned, inconsistent) */
  PSATTN_E_UNSUPPORTED = 2,  /* well-formed but outside the supported set (no fallback is run) */
  PSATTN_E_WORKSPACE = 3,    /* workspace missing or smaller than psattn_workspace_size() */
  PSATTN_E_HIP = 4           /* a HIP runtime call failed while enqueuing */
} psattn_status;

enum { PSATTN_MODE_FLAT = 0, PSATTN_MODE_PAGED = 1 };

/*
 * Segment descriptor.  Device arrays are borrowed until the enqueued work
 * has finished.
 *
 * Flat mode (GRPO rollouts sharing one prompt):
 *   q, o      [total_tokens, Hq, D]  row-major, packed [P | S1 | ... | SN]
 *   k, v      [total_tokens, Hkv, D]
 *   lse       [total_tokens, Hq]     fp32
 *   seg_offsets (device, int32, num_segments + 1 entries): seg_offsets[0] =
 *     prefix_len, seg_offsets[num_segments] = total_tokens, non-decreasing.
 *     Empty segments are allowed.  num_segments = 0 means the buffer holds the
 *     prefix alone (then total_tokens == prefix_len and seg_offsets may be NULL).
 *   max_seg_len (host): a bound of the segment lengths, checked on the host
 *     only as num_segments * max_seg_len >= total_tokens - prefix_len.  The
 *     forward does not use it; the backward sizes its dK/dV launch from it,
 *     and a value below the true longest segment costs time there (the
 *     workgroups walk the surplus items), never correctness.
 *   seg_parent (device, int32, num_segments entries) or NULL: multi-level
 *     sharing (the multi-level tree "chain" case that the PrefixSharing PR #50
 *     page lists beside the flat GRPO case in its mask-construction section,
 *     and plans as "multi-level tree support": rollouts that share a common
 *     continuation of the prompt as well as the prompt).  seg_parent[i] = -1
 *     means segment i continues the prefix
 *     directly; otherwise seg_parent[i] = j with 0 <= j < i, and segment i
 *     continues segment j.  A row of segment i then sees the prefix, every
 *     token of each ancestor segment (j, its parent, ... up to the prefix),
 *     and its own segment causally: ordinary causal attention over
 *     [P | ancestors, root-most first | S_i].  Entries outside [-1, i) end
 *     the ancestor walk there (no out-of-bounds read, no endless loop, but
 *     those rows are then wrong).  NULL: one level (every parent is -1).
 *     bf16 only (forward and psattn_bwd); ignored in paged mode.
 *
 * Paged mode (speculative target-verify; draft_len rows per request, or
 * ragged lengths through qo_indptr):
 *   q, o      [batch * draft_len, Hq, D]; draft row t of request b is row
 *             b * draft_len + t and sits at position prefix_lens[b] + t.
 *   lse       [batch * draft_len, Hq]   fp32
 *   k, v      page pools [num_pages, page_size, Hkv, D] in kv dtype; any
 *             page_size >= 1 (the sglang PR #27382 report, "关键源码片段",
 *             addresses its k_buffer / v_buffer through kv_indptr / kv_indices
 *             without fixing a page size)
 *   kv_indptr (device, int32, batch + 1): request b owns the page ids
 *             kv_indices[kv_indptr[b] .. kv_indptr[b+1]); prefix token t of b
 *             is slot t % page_size of page kv_indices[kv_indptr[b] + t / page_size].
 *             kv_indptr[b+1] - kv_indptr[b] >= ceil(prefix_lens[b] / page_size).
 *   prefix_lens (device, int32, batch): 0 <= prefix_lens[b] <= max_prefix_len.
 *   max_prefix_len (host): upper bound of prefix_lens (sizes the split grid).
 *   k_ext, v_ext [batch * draft_len, Hkv, D] in kv dtype: the draft block's own
 *             K/V; draft row t sees draft keys 0..t, or, with draft_mask,
 *             the draft keys its mask row marks.
 *   draft_mask (device, uint8, [batch, draft_len, draft_len]) or NULL: a draft
 *             tree (EAGLE top-k > 1; the sglang verify page's custom mask over
 *             the draft part, prefix part skipped): draft row t of request b
 *             sees draft key j iff draft_mask[(b * draft_len + t) * draft_len
 *             + j] != 0, and every prefix key.  Each row must see itself (a
 *             tree row holds its ancestors and its own token).  NULL: the
 *             causal chain.  Ignored in flat mode.  With qo_indptr the mask
 *             keeps this padded layout; request b uses its first n_b rows and
 *             columns.
 *   qo_indptr (device, int32, batch + 1) or NULL: ragged draft lengths.
 *             Request b's draft rows of q, o, lse, k_ext and v_ext are
 *             qo_indptr[b] .. qo_indptr[b+1] (n_b of them, 0 <= n_b <=
 *             draft_len, which is then the upper bound); draft row t sits at
 *             position prefix_lens[b] + t.  NULL: n_b = draft_len for every
 *             request and its rows start at b * draft_len.
 */
typedef struct {
  int32_t mode;
  /* flat */
  int64_t total_tokens;
  int32_t prefix_len;
  int32_t num_segments;
  const int32_t* seg_offsets;
  int32_t max_seg_len;
  /* paged */
  int32_t batch;
  int32_t draft_len;
  int32_t page_size;
  int32_t num_pages;
  const int32_t* prefix_lens;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int32_t max_prefix_len;
  const void* k_ext;
  const void* v_ext;
  const uint8_t* draft_mask;
  const int32_t* qo_indptr;
  /* flat, multi-level sharing */
  const int32_t* seg_parent;
} psattn_desc;

/*
 * Launch plan summary (host struct) reported by psattn_plan_dump /
 * psattn_plan_host.  n_items is the number of workgroups the forward launch
 * of the prefix pass uses (one work item each, idle ones included).
 */
typedef struct {
  int64_t n_items;
  int32_t tile_tokens;     /* flat: query tokens per tile (rows per tile / G) */
  int32_t rows_per_tile;   /* stacked query rows (tokens x GQA heads) per workgroup */
  int32_t n_splits;        /* paged: splits per (request, kv head) */
  int32_t split_len;       /* paged: prefix tokens per split (multiple of page_size) */
  int32_t kv_tile;         /* keys per inner-loop tile */
  int32_t reserved;
} psattn_plan_info;

/* Work-item record written by the planner: 10 int32 per item, in this order. */
enum {
  PSATTN_ITEM_FIELDS = 10,
  PSATTN_ITEM_NONE = 0,        /* idle workgroup */
  PSATTN_ITEM_FLAT_PREFIX = 1, /* tile of prefix rows */
  PSATTN_ITEM_FLAT_SUFFIX = 2, /* tile of one rollout's rows */
  PSATTN_ITEM_PAGED_SPLIT = 3  /* one split of one request's prefix, one kv head */
};
/* fields: kind, h_kv, seg (flat: rollout index or -1; paged: request),
 *         q_begin, q_end (flat: packed rows; paged: draft rows 0..draft_len),
 *         r0_begin, r0_end, r1_begin, r1_end (key ranges; a flat row r sees
 *         (r0 U r1) intersected with [0, r]; a paged split covers prefix keys r0),
 *         split. */

/*
 * Bytes of scratch the forward call needs for this descriptor (0 in flat
 * mode; paged mode: per-split partial O (bf16 for the streaming split
 * passes that serve bf16 and fp8 caches in pages of >= 16 slots with up to
 * 64 stacked rows, fp32 otherwise) and its LSE in fp32, the first stage's
 * output that the second stage merges, sglang PR #27382 report, "实现拆解").
 * The caller owns this memory and passes it to every call, so the library
 * keeps no buffer of its own between calls (that report's review section,
 * "评论区精华", describes split scratch buffers cached under the batch size,
 * one allocation per batch size seen, which bloated device memory).  The
 * size is a pure function of the descriptor's host fields and the shapes.
 * Host only; does not touch the GPU.  Returns 0 and sets the last error on
 * invalid input.
 */
size_t psattn_workspace_size(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                             psattn_dtype q_dtype, psattn_dtype kv_dtype);

/*
 * Forward pass (flat: one launch; paged: split pass + combine pass).
 *   q, k, v, o, lse : device pointers, 16-byte aligned, layouts as above.
 *   hq, hkv, d      : heads and head dim; hq % hkv == 0; d in {64, 128, 256}.
 *   sm_scale        : logit scale (> 0), e.g. 1/sqrt(d).
 *   q_dtype/kv_dtype: supported pairs (F32,F32) and (BF16,BF16) in both modes,
 *                     (BF16,FP8_E4M3) in paged mode. o has q's dtype.
 *   k_scale,v_scale : per-tensor multipliers of stored K and V (paged mode;
 *                     must be 1 in flat mode).
 *   workspace       : device scratch of at least psattn_workspace_size() bytes
 *                     (may be NULL when that size is 0), 256-byte aligned.
 *   stream          : hipStream_t.
 * Returns PSATTN_OK once the work is enqueued.
 */
psattn_status psattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                         float sm_scale, psattn_dtype q_dtype, psattn_dtype kv_dtype,
                         float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory at
 * call time (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): psattn_fwd with the paged split scratch taken from
 * a fixed array of PSATTN_NOALLOC_SCRATCH_BYTES in device memory, one per GPU,
 * instead of a caller workspace.  Arguments, layouts, results and errors are
 * those of psattn_fwd; a descriptor whose psattn_workspace_size() exceeds
 * PSATTN_NOALLOC_SCRATCH_BYTES returns PSATTN_E_UNSUPPORTED with nothing
 * enqueued.  The call allocates and frees nothing; the array used is that of
 * the stream's device, whose address the first call on that device looks up
 * once (making the device current for the lookup only).  Every call on one GPU shares
 * its array (the contents on entry do not matter, each call writes what it
 * reads), so calls that overlap on one GPU -- on two streams, or from two
 * threads without ordering -- race and give undefined results.
 */
#define PSATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
psattn_status psattn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                                 float sm_scale, psattn_dtype q_dtype, psattn_dtype kv_dtype,
                                 float k_scale, float v_scale, void* stream);

/*
 * Backward of the flat forward (PrefixSharing PR #50, "关键变更" / key
 * changes: the rollouts' KV is built by copying the prefix with .copy_(), so
 * gradients flow back through the copies and a stored prefix row receives the
 * sum of all its copies' gradients; equivalently, the gradient of one
 * attention over the flat buffer with the block-causal visibility).  The
 * flat output's prefix rows count once.
 *
 * Bytes of scratch psattn_bwd needs (flat mode only): lse2 and delta, [T, Hq]
 * fp32 each, fp32 dK / dV accumulators, [T, Hkv, D] each, and a table of
 * the key-major pass's work items (16 bytes each, as many as the host's bound
 * on one kv head's items from the descriptor's scalars, plus one entry for
 * the first item past that bound).  Host only.
 * Returns 0 and sets the last error on invalid or unsupported input.
 */
size_t psattn_bwd_workspace_size(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                                 psattn_dtype dtype);

/*
 * Gradients dQ, dK, dV of the flat forward for the upstream gradient dO.
 *   q, k, v, o   : the forward's inputs and output ([T, Hq, D], [T, Hkv, D],
 *                  [T, Hkv, D], [T, Hq, D]); device, 16-byte aligned.
 *   lse          : the forward's LSE [T, Hq], fp32, natural log.
 *   dout         : dO [T, Hq, D], q's dtype.
 *   dq, dk, dv   : outputs, layouts of q, k, v, in q's dtype; fully written.
 *   desc         : flat descriptor (mode PSATTN_MODE_FLAT), as for psattn_fwd,
 *                  seg_parent included: with it, the gradient of the
 *                  multi-level forward (each segment's expansion copies the
 *                  prefix and its ancestors' tokens, and every copy's gradient
 *                  flows back to the stored row).
 *   d            : 64, 128 or 256.  dtype: PSATTN_BF16.  hq / hkv <= 64.
 *   sm_scale     : the forward's logit scale.
 *   workspace    : device scratch of psattn_bwd_workspace_size() bytes,
 *                  256-byte aligned; its contents on entry do not matter.
 * Enqueues four launches on `stream` (dQ, which also forms the row terms,
 * zeroes the accumulators and writes the item table; dK/dV over the items
 * that max_seg_len predicts; dK/dV over any items past that bound; and the
 * conversion; at d = 256 the two dK/dV launches run once per half of the
 * head dimension).
 * dK and dV sum fp32 partials with atomic adds, so their last bits may
 * differ between calls; dQ is deterministic.  Other configurations return
 * PSATTN_E_UNSUPPORTED with nothing enqueued.
 */
psattn_status psattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, const psattn_desc* desc,
                         int32_t hq, int32_t hkv, int32_t d, float sm_scale, psattn_dtype dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse shared-latent MLA forward (DSA / sparse-MLA prefill; the vLLM issue
 * "[Perf] SM8x sparse-MLA prefill fallback re-reads the shared MLA latent
 * once per head", sections 适用环境 and 原因分析): every query token attends
 * to the cached tokens its top-k list names, and all of its heads read the
 * same latent rows, which serve as keys and values (the NoPE layout,
 * kv_lora_rank = 512, no rope part).  One workgroup stacks all heads of a
 * token, so each gathered latent row is read once per token, not per head.
 *   q       : [num_tokens, num_heads, dim] bf16, device, 16-byte aligned.
 *   ckv     : the latent cache, num_kv rows of kv_stride bf16 elements (the
 *             first dim used), device, 16-byte aligned; the buffer must hold
 *             (num_kv - 1) * kv_stride + dim elements.
 *   indices : [num_tokens, topk] int32, device: cache rows token t attends
 *             to, once per entry (an entry listed twice counts twice).
 *             Entries outside [0, num_kv), such as -1 padding, are skipped.
 *   sink    : [num_heads] fp32 natural-log logits, device, or NULL: sink_h
 *             joins head h's softmax normaliser and carries no value.
 *   o, lse  : outputs [num_tokens, num_heads, dim] bf16 and [num_tokens,
 *             num_heads] fp32 (natural log).  o[t, h] = sum_j e^{z_j} c_j /
 *             (sum_j e^{z_j} + e^{sink_h}), z_j = sm_scale <q[t, h], c_j>,
 *             lse = ln of that denominator.  A token with no valid entry
 *             gets o = 0 and lse = sink_h, or -inf without sinks.
 *   dim = 512; num_heads in {32, 64, 128}; 0 <= topk <= 2048; kv_stride >=
 *   dim, a multiple of 8; dtype PSATTN_BF16.  Allocates nothing; one launch
 *   on `stream`.  Other configurations return PSATTN_E_UNSUPPORTED or
 *   PSATTN_E_INVAL with nothing enqueued.
 */
psattn_status psattn_mla_fwd(const void* q, const void* ckv, const int32_t* indices, const float* sink, void* o,
                             float* lse, int64_t num_tokens, int32_t num_heads, int32_t dim, int64_t num_kv,
                             int32_t kv_stride, int32_t topk, float sm_scale, psattn_dtype dtype, void* stream);

/*
 * Dense causal shared-latent MLA prefill: the same head-stacked latent
 * attention with no list (the shared-latent MLA of that page with every
 * earlier cached row visible).  The num_tokens query tokens are the last
 * num_tokens rows of the cache: token t sits at row num_kv - num_tokens + t
 * and attends to rows 0 .. num_kv - num_tokens + t, in order.  Arguments,
 * layouts, sink, outputs and limits as for psattn_mla_fwd without indices
 * and topk; num_kv >= num_tokens (else PSATTN_E_INVAL).  Allocates nothing;
 * one launch on `stream`.
 */
psattn_status psattn_mla_dense_fwd(const void* q, const void* ckv, const float* sink, void* o, float* lse,
                                   int64_t num_tokens, int32_t num_heads, int32_t dim, int64_t num_kv,
                                   int32_t kv_stride, float sm_scale, psattn_dtype dtype, void* stream);

/*
 * Test hook: run the segment planner ON THE DEVICE for every workgroup of the
 * prefix-pass launch psattn_fwd would make and write its work items (the
 * PrefixSharing PR #50 page, "设计简介", proposes describing the visibility
 * by rectangles instead of a dense mask; the items are those rectangles)
 * (PSATTN_ITEM_FIELDS int32 each, in workgroup order) to items_dev, which
 * must hold `capacity` items.  info_host (host) receives the plan summary.
 * With items_dev == NULL only info_host is filled (no GPU work).
 */
psattn_status psattn_plan_dump(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                               psattn_dtype q_dtype, psattn_dtype kv_dtype, int32_t* items_dev,
                               int64_t capacity, psattn_plan_info* info_host, void* stream);

/*
 * Same planner code run on the host: the descriptor's arrays (seg_offsets,
 * prefix_lens) are HOST pointers here and items_host is a host buffer.
 */
psattn_status psattn_plan_host(const psattn_desc* desc, int32_t hq, int32_t hkv, int32_t d,
                               psattn_dtype q_dtype, psattn_dtype kv_dtype, int32_t* items_host,
                               int64_t capacity, psattn_plan_info* info_host);

/* Static description of a status code. */
const char* psattn_status_string(psattn_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* psattn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PSATTN_H_ */
