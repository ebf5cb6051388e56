// mla.h -- internal interface of the shared-latent MLA forward (sparse top-k
// lists or dense causal).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace psattn {

constexpr int kMlaDim = 512;        // latent width (kv_lora_rank)
constexpr int kMlaMaxTopk = 2048;   // index entries per token staged in LDS

struct MlaArgs {
  const void* q;           // [T, H, 512] bf16
  const void* ckv;         // [S] rows of kv_stride bf16, the first 512 used
  const int32_t* indices;  // [T, topk], or null (dense)
  const float* sink;       // [H] natural-log sink logits, or null
  void* o;                 // [T, H, 512] bf16
  float* lse;              // [T, H] fp32, natural log
  int32_t num_tokens;
  int32_t num_heads;
  int32_t num_kv;
  int32_t kv_stride;       // elements between latent rows
  int32_t topk;
  float scale_log2;        // sm_scale * log2(e)
};

// dense: no list (indices null); token t takes cache rows 0 .. num_kv - num_tokens + t
int launch_mla(const MlaArgs& a, bool dense, void* stream);

}  // namespace psattn
