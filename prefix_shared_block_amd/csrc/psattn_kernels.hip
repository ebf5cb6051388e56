// psattn_kernels.hip -- gfx950 kernels for prefix-shared attention forward.
//
// Three kernels:
//  * flat_fwd     one launch for the flat-packed GRPO layout [P | S1..SN]
//                 (PrefixSharing PR #50, "设计简介"): each workgroup takes one
//                 planner tile of stacked query rows (tokens x GQA heads of one
//                 kv head), streams the prefix K/V tiles and then its own
//                 rollout's K/V tiles through LDS, and finishes the softmax.
//  * paged_split  split-KV prefix pass for speculative verify (sglang PR
//                 #27382, "实现拆解", first stage): per (request, kv head,
//                 split) a partial output and log-sum-exp, fp8 K/V decoded to
//                 bf16 on the way into LDS with k_scale folded into the logit
//                 scale.
//  * paged_combine  second stage: log-sum-exp merge of the splits together
//                 with the causal draft-by-draft block, v_scale applied.
//
// Shared tile engine (one wave = 32 stacked query rows):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys from LDS, B = the
//   wave's Q rows kept in registers), so a lane holds 16 scores of ONE query
//   row; row max / row sum are lane-local plus one swap with lane l^32.
//   The score accumulator is, unchanged, the B operand of O^T = V^T P^T, so
//   the output accumulator is also indexed by the lane's own query and the
//   online-softmax rescale is lane-local.  V is written transposed into LDS
//   so that the A operand (8 keys of one d column) is two 8-byte reads.
//   fp32 inputs use v_mfma_f32_32x32x2f32 with the same layouts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace psattn {

// ---------------------------------------------------------------------------
// LDS tile geometry.  bf16 compute: K row-major [BN][D+8], V transposed
// [D][BN+4].  fp32 compute: K and V row-major [BN][D+4].
// ---------------------------------------------------------------------------
template <int D, bool F32C, int BN>
struct Lds {
  static constexpr int KSTR = D + (F32C ? 4 : 8);
  static constexpr int VSTR = F32C ? (D + 4) : (BN + 4);
  static constexpr int CS = F32C ? 4 : 2;
  static constexpr int KBYTES = BN * KSTR * CS;
  static constexpr int VBYTES = F32C ? BN * VSTR * 4 : D * VSTR * 2;
  static constexpr int BYTES = KBYTES + VBYTES;
};

// ---------------------------------------------------------------------------
// Cooperative tile loader: BN keys x D, 256 threads, 16-byte global reads.
// Thread t owns chunk c = t % CPR of RPT consecutive key rows, so each load
// instruction of a wave reads whole rows; V rows of one thread are then
// written transposed as packed key pairs.
// ---------------------------------------------------------------------------
template <int KDT, int D, int BN, bool PAGED>
struct TileLoader {
  static constexpr int ES = Elem<KDT>::size;
  static constexpr int CPR = D * ES / 16;
  static constexpr int RG = kThreads / CPR;
  static constexpr int RPT = (BN / RG) > 0 ? (BN / RG) : 1;
  static constexpr int EPC = 16 / ES;  // elements per 16-byte chunk
  static constexpr bool F32C = (KDT == DT_F32);
  using L = Lds<D, F32C, BN>;

  u32x4_t kr[RPT];
  u32x4_t vr[RPT];
  int c;
  int rgrp;
  bool active;

  __device__ void init(int tid) {
    c = tid % CPR;
    rgrp = tid / CPR;
    active = rgrp * RPT < BN;
  }

  // flat: rows are token indices of the packed [T, Hkv, D] tensors
  __device__ void load_flat(const char* kbase, const char* vbase, int hkv, int h_kv, int key0,
                            int kend) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      int key = key0 + rgrp * RPT + i;
      key = key < kend ? key : kend - 1;
      size_t off = (((size_t)key * hkv + h_kv) * D) * ES + (size_t)c * 16;
      kr[i] = *reinterpret_cast<const u32x4_t*>(kbase + off);
      vr[i] = *reinterpret_cast<const u32x4_t*>(vbase + off);
    }
  }

  // paged: rows are prefix positions of one request, looked up page by page
  __device__ void load_paged(const char* kpool, const char* vpool, const int32_t* pages,
                             int page_size, int hkv, int h_kv, int key0, int kend) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      int key = key0 + rgrp * RPT + i;
      key = key < kend ? key : kend - 1;
      int pg = pages[key / page_size];
      int slot = key - (key / page_size) * page_size;
      size_t row = ((size_t)pg * page_size + slot) * hkv + h_kv;
      size_t off = row * D * ES + (size_t)c * 16;
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kpool + off));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vpool + off));
    }
  }

  __device__ void store(char* lds) {
    if (!active) return;
    if constexpr (F32C) {
      float* kl = reinterpret_cast<float*>(lds);
      float* vl = reinterpret_cast<float*>(lds + L::KBYTES);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        int r = rgrp * RPT + i;
        *reinterpret_cast<u32x4_t*>(kl + r * L::KSTR + c * 4) = kr[i];
        *reinterpret_cast<u32x4_t*>(vl + r * L::VSTR + c * 4) = vr[i];
      }
    } else {
      __bf16* kl = reinterpret_cast<__bf16*>(lds);
      __bf16* vt = reinterpret_cast<__bf16*>(lds + L::KBYTES);
      constexpr int ECH = (KDT == DT_FP8) ? 16 : 8;  // bf16 elements per thread chunk
      u32x4_t kb[RPT][ECH / 8];
      u32x4_t vb[RPT][ECH / 8];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        if constexpr (KDT == DT_FP8) {
          fp8x16_to_bf16(kr[i], kb[i][0], kb[i][ECH / 8 - 1]);
          fp8x16_to_bf16(vr[i], vb[i][0], vb[i][ECH / 8 - 1]);
        } else {
          kb[i][0] = kr[i];
          vb[i][0] = vr[i];
        }
      }
      const int d0 = c * ECH;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        int r = rgrp * RPT + i;
#pragma unroll
        for (int h = 0; h < ECH / 8; ++h)
          *reinterpret_cast<u32x4_t*>(kl + r * L::KSTR + d0 + 8 * h) = kb[i][h];
      }
      // V^T: element e of the chunk goes to row d0 + e, keys rgrp*RPT .. +RPT
      const int k0 = rgrp * RPT;
#pragma unroll
      for (int e = 0; e < ECH; ++e) {
        __bf16* dst = vt + (d0 + e) * L::VSTR + k0;
        if constexpr (RPT == 1) {
          uint16_t x = (uint16_t)half_of(vb[0][e >> 3], e & 7);
          *reinterpret_cast<uint16_t*>(dst) = x;
        } else {
          // key pairs packed into dwords, written 8 bytes (two pairs) at a time
#pragma unroll
          for (int q2 = 0; q2 < RPT / 2; q2 += 2) {
            const uint32_t w0 = half_of(vb[2 * q2][e >> 3], e & 7) |
                                (half_of(vb[2 * q2 + 1][e >> 3], e & 7) << 16);
            if (q2 + 1 < RPT / 2) {
              const uint32_t w1 = half_of(vb[2 * q2 + 2][e >> 3], e & 7) |
                                  (half_of(vb[2 * q2 + 3][e >> 3], e & 7) << 16);
              u32x2_t w = {w0, w1};
              *reinterpret_cast<u32x2_t*>(dst + 2 * q2) = w;
            } else {
              *reinterpret_cast<uint32_t*>(dst + 2 * q2) = w0;
            }
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Per-wave query fragment and online-softmax state
// ---------------------------------------------------------------------------
template <int D, bool F32C>
struct QFrag;
template <int D>
struct QFrag<D, false> {
  bf16x8_t v[D / 16];  // step ks: d = h*D/2 + 8ks .. +8
  __device__ void load(const __bf16* row, int h) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(row + h * (D / 2));
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) v[ks] = __builtin_bit_cast(bf16x8_t, p[ks]);
  }
};
template <int D>
struct QFrag<D, true> {
  float v[D / 2];  // step s: d = h*D/2 + s
  __device__ void load(const float* row, int h) {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(row + h * (D / 2));
#pragma unroll
    for (int s4 = 0; s4 < D / 8; ++s4) {
      f32x4_t x = p[s4];
      v[4 * s4 + 0] = x[0];
      v[4 * s4 + 1] = x[1];
      v[4 * s4 + 2] = x[2];
      v[4 * s4 + 3] = x[3];
    }
  }
};

template <int D>
struct WaveState {
  f32x16_t o[D / 32];  // O^T: lane (c,h) holds d = 32db + 8(i/4) + 4h + i%4 of query c
  float m;             // running max (log2 domain), equal in lanes c and c+32
  float l;             // this lane's partial row sum (lanes c and c+32 add up)
  __device__ void init() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    m = kNegBig;
    l = 0.f;
  }
};

// One wave consumes BNW keys (LDS rows koff .. koff+BNW) against its 32 rows.
// key0: global key index of LDS row koff; kend: first invisible key of the
// range; token: the lane's query position (causal limit), INT_MAX if none.
template <int D, bool F32C, int BN, int BNW>
__device__ __forceinline__ void process_tile(WaveState<D>& st, const QFrag<D, F32C>& qf,
                                             const char* lds, int koff, int key0, int kend,
                                             int token, bool needmask, float scale_log2) {
  using L = Lds<D, F32C, BN>;
  constexpr int NKB = BNW / 32;
  const int lane = __lane_id();
  const int c = lane & 31;
  const int h = lane >> 5;
  f32x16_t s[NKB];

  // ---- scores S^T = K Q^T
  if constexpr (!F32C) {
    const __bf16* kl = reinterpret_cast<const __bf16*>(lds);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const __bf16* kp = kl + (koff + kb * 32 + c) * L::KSTR + h * (D / 2);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + 8 * ks);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.v[ks], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }
  } else {
    const float* kl = reinterpret_cast<const float*>(lds);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const float* kp = kl + (koff + kb * 32 + c) * L::KSTR + h * (D / 2);
#pragma unroll
      for (int s4 = 0; s4 < D / 8; ++s4) {
        f32x4_t a = *reinterpret_cast<const f32x4_t*>(kp + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf.v[4 * s4 + e], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }
  }

  // ---- online softmax (log2 domain)
  float mx = kNegBig;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = s[kb][i] * scale_log2;
      if (needmask) {
        int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= kend || key > token) x = -__builtin_inff();
      }
      s[kb][i] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, swap_halves(mx));
  const float m_new = fmaxf(st.m, mx);
  const float alpha = fast_exp2(st.m - m_new);
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = fast_exp2(s[kb][i] - m_new);
      s[kb][i] = p;
      psum += p;
    }
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;

  // ---- O^T += V^T P^T
  if constexpr (!F32C) {
    const __bf16* vt = reinterpret_cast<const __bf16*>(lds + L::KBYTES);
#pragma unroll
    for (int kstep = 0; kstep < BNW / 16; ++kstep) {
      const int kb = kstep >> 1;
      const int base = 8 * (kstep & 1);
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kb][base + e];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const __bf16* vp = vt + (db * 32 + c) * L::VSTR + koff + 16 * kstep + 4 * h;
        bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(vp);
        bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(vp + 8);
        bf16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, st.o[db], 0, 0, 0);
      }
    }
  } else {
    const float* vl = reinterpret_cast<const float*>(lds + L::KBYTES);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = koff + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          float a = vl[key * L::VSTR + db * 32 + c];
          st.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][i], st.o[db], 0, 0, 0);
        }
      }
    }
  }
}

// store 4 consecutive output elements
template <bool F32C>
__device__ __forceinline__ void store4(void* base, size_t idx, float a, float b, float c, float d) {
  if constexpr (F32C) {
    f32x4_t v = {a, b, c, d};
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + idx) = v;
  } else {
    u32x2_t v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<__bf16*>(base) + idx) = v;
  }
}

// ===========================================================================
// Flat (GRPO) kernel
// ===========================================================================
template <int D, bool F32C>
struct FlatCfg {
  static constexpr int BN = D >= 256 ? 32 : 64;
  using L = Lds<D, F32C, BN>;
  static constexpr int NBUF = 2;
  static constexpr int MINB = (D >= 256 || (F32C && D >= 128)) ? 1 : 2;
};

template <int D, bool F32C>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FlatCfg<D, F32C>::MINB)))
void flat_fwd_kernel(FlatArgs a) {
  using Cfg = FlatCfg<D, F32C>;
  using L = typename Cfg::L;
  constexpr int BN = Cfg::BN;
  constexpr int KDT = F32C ? DT_F32 : DT_BF16;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::NBUF * L::BYTES];

  const int blk = blockIdx.x;
  const int h_kv = blk % a.hkv;
  const int j = blk / a.hkv;
  const Item it = flat_item(j, h_kv, a.prefix_len, a.nseg, a.seg_offsets, a.tile_tokens);
  if (it.kind == kNone) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;

  // stacked row of this lane's query column: token-major, heads interleaved
  const int r = wave * kWaveRows + c;
  const int tok = r / a.g;
  const int hl = r - tok * a.g;
  const int token = it.q_begin + tok;
  const bool valid = (tok < a.tile_tokens) && (token < it.q_end);
  const int token_c = valid ? token : it.q_begin;
  const int head = h_kv * a.g + hl;
  const size_t qrow = (size_t)token_c * a.hq + head;

  QFrag<D, F32C> qf;
  if constexpr (F32C)
    qf.load(reinterpret_cast<const float*>(a.q) + qrow * D, h);
  else
    qf.load(reinterpret_cast<const __bf16*>(a.q) + qrow * D, h);

  WaveState<D> st;
  st.init();

  TileLoader<KDT, D, BN, false> ld;
  ld.init(tid);
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);

  const int n0 = cdiv32(it.r0_end - it.r0_begin, BN);
  const int n1 = cdiv32(it.r1_end - it.r1_begin, BN);
  const int nt = n0 + n1;

  auto tile_range = [&](int n, int& k0, int& ke) {
    if (n < n0) {
      k0 = it.r0_begin + n * BN;
      ke = it.r0_end;
    } else {
      k0 = it.r1_begin + (n - n0) * BN;
      ke = it.r1_end;
    }
  };

  int k0, ke;
  tile_range(0, k0, ke);
  ld.load_flat(kbase, vbase, a.hkv, h_kv, k0, ke);
  ld.store(smem);
  __syncthreads();

  for (int n = 0; n < nt; ++n) {
    int cur_k0, cur_ke;
    tile_range(n, cur_k0, cur_ke);
    if (n + 1 < nt) {
      int nk0, nke;
      tile_range(n + 1, nk0, nke);
      ld.load_flat(kbase, vbase, a.hkv, h_kv, nk0, nke);
    }
    const bool needmask = (cur_k0 + BN > cur_ke) || (cur_k0 + BN - 1 > it.q_begin);
    process_tile<D, F32C, BN, BN>(st, qf, smem + (n & 1) * L::BYTES, 0, cur_k0, cur_ke, token,
                                  needmask, a.scale_log2);
    if (n + 1 < nt) ld.store(smem + ((n + 1) & 1) * L::BYTES);
    __syncthreads();
  }

  // ---- epilogue
  const float lt = st.l + swap_halves(st.l);
  const float inv = 1.0f / lt;
  if (valid) {
    const size_t obase = qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * h;
        store4<F32C>(a.o, obase + d, st.o[db][4 * g4] * inv, st.o[db][4 * g4 + 1] * inv,
                     st.o[db][4 * g4 + 2] * inv, st.o[db][4 * g4 + 3] * inv);
      }
    }
    if (h == 0) a.lse[qrow] = (st.m + fast_log2(lt)) * kLn2;
  }
}

// ===========================================================================
// Paged split-KV prefix pass
// ===========================================================================
template <int D, int KDT, int RB>
struct PagedCfg {
  static constexpr bool F32C = (KDT == DT_F32);
  static constexpr int KS = kWaves / RB;
  static constexpr int BN = KS * 32;
  using L = Lds<D, F32C, BN>;
  static constexpr int MERGE_FLOATS = (KS - 1) * RB * 64 * (16 * (D / 32) + 2);
  static constexpr int SMEM = (L::BYTES > MERGE_FLOATS * 4) ? L::BYTES : MERGE_FLOATS * 4;
  static constexpr int MINB = (D >= 256 || (F32C && D >= 128)) ? 1 : 2;
};

template <int D, int KDT, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PagedCfg<D, KDT, RB>::MINB)))
void paged_split_kernel(PagedArgs a) {
  using Cfg = PagedCfg<D, KDT, RB>;
  using L = typename Cfg::L;
  constexpr bool F32C = Cfg::F32C;
  constexpr int KS = Cfg::KS;
  constexpr int BN = Cfg::BN;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::SMEM];

  const Item it = paged_item(blockIdx.x, a.hkv, a.n_splits, a.split_len, a.draft_len,
                             a.prefix_lens);
  const int b = it.seg;
  const int h_kv = it.h_kv;
  const int qbase = draft_base(a.qo_indptr, b, a.draft_len);  // the request's first draft row
  const int qn = draft_count(a.qo_indptr, b, a.draft_len);    // and its number of draft rows
  if (qn <= 0) return;                                         // a request without draft rows

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;
  const int rb = wave % RB;
  const int ks = wave / RB;

  const int r = rb * kWaveRows + c;  // stacked row: draft-token-major, heads interleaved
  const bool valid = r < a.rows && r / a.g < qn;
  const int rc = valid ? r : 0;
  const int t = rc / a.g;
  const int hl = rc - t * a.g;
  const size_t qrow = (size_t)(qbase + t) * a.hq + h_kv * a.g + hl;

  QFrag<D, F32C> qf;
  if constexpr (F32C)
    qf.load(reinterpret_cast<const float*>(a.q) + qrow * D, h);
  else
    qf.load(reinterpret_cast<const __bf16*>(a.q) + qrow * D, h);

  WaveState<D> st;
  st.init();

  TileLoader<KDT, D, BN, true> ld;
  ld.init(tid);
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const int32_t* pages = a.kv_indices + a.kv_indptr[b];

  const int kend = it.r0_end;
  const int nt = cdiv32(it.r0_end - it.r0_begin, BN);
  constexpr int NOMASK_TOKEN = 0x7fffffff;

  if (nt > 0) {
    ld.load_paged(kpool, vpool, pages, a.page_size, a.hkv, h_kv, it.r0_begin, kend);
    ld.store(smem);
    __syncthreads();
  }
  for (int n = 0; n < nt; ++n) {
    const int k0 = it.r0_begin + n * BN;
    if (n + 1 < nt)
      ld.load_paged(kpool, vpool, pages, a.page_size, a.hkv, h_kv, k0 + BN, kend);
    const int wk0 = k0 + ks * 32;
    if (wk0 < kend) {
      const bool needmask = wk0 + 32 > kend;
      process_tile<D, F32C, BN, 32>(st, qf, smem, ks * 32, wk0, kend, NOMASK_TOKEN, needmask,
                                    a.scale_log2);
    }
    __syncthreads();
    if (n + 1 < nt) {
      ld.store(smem);
      __syncthreads();
    }
  }

  // ---- merge the key streams of each row block through LDS
  constexpr int NV = 16 * (D / 32) + 2;
  if constexpr (KS > 1) {
    float* mb = reinterpret_cast<float*>(smem);
    if (ks > 0) {
      float* dst = mb + (((ks - 1) * RB + rb) * 64 + lane) * NV;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[db * 16 + i] = st.o[db][i];
      dst[NV - 2] = st.m;
      dst[NV - 1] = st.l;
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int o = 1; o < KS; ++o) {
        const float* src = mb + (((o - 1) * RB + rb) * 64 + lane) * NV;
        const float m2 = src[NV - 2];
        const float l2 = src[NV - 1];
        const float mn = fmaxf(st.m, m2);
        const float a1 = fast_exp2(st.m - mn);
        const float a2 = fast_exp2(m2 - mn);
        st.l = st.l * a1 + l2 * a2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) st.o[db][i] = st.o[db][i] * a1 + src[db * 16 + i] * a2;
        st.m = mn;
      }
    }
  }
  if (ks != 0) return;

  // ---- partial output for this split: O_s = acc / l, LSE_s = m + log2 l
  const float lt = st.l + swap_halves(st.l);
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  if (valid) {
    const size_t prow = (((size_t)b * a.hkv + h_kv) * a.n_splits + it.split) * a.rows + r;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * h;
        f32x4_t v = {st.o[db][4 * g4] * inv, st.o[db][4 * g4 + 1] * inv,
                     st.o[db][4 * g4 + 2] * inv, st.o[db][4 * g4 + 3] * inv};
        *reinterpret_cast<f32x4_t*>(po + d) = v;
      }
    }
    if (h == 0) a.part_lse[prow] = empty ? -__builtin_inff() : st.m + fast_log2(lt);
  }
}

// ===========================================================================
// Combine: merge splits by log-sum-exp and fold in the causal draft block.
// One wave per (request, kv head, stacked row).
// ===========================================================================
// One wave per (request, kv head, stacked row, 64-column chunk of the head
// dimension): the draft-block logits need the full head dimension (each wave
// recomputes them; they are tiny), the merge touches only the wave's chunk.
template <int D, int QDT, int KDT>
__global__ __launch_bounds__(256) void paged_combine_kernel(PagedArgs a, float scale_log2_draft) {
  constexpr int PER = D / 64;  // d elements per lane for the dot products: d = lane + 64 * e
  const int gw = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * 256 + threadIdx.x) >> 6));
  const int lane = threadIdx.x & 63;
  const int total = a.batch * a.hkv * a.rows * PER;
  if (gw >= total) return;
  const int chunk = gw % PER;
  const int wave = gw / PER;
  const int r = wave % a.rows;
  const int h_kv = (wave / a.rows) % a.hkv;
  const int b = wave / (a.rows * a.hkv);
  const int t = r / a.g;
  const int hl = r - t * a.g;
  const int head = h_kv * a.g + hl;
  const int qbase = draft_base(a.qo_indptr, b, a.draft_len);
  const int qn = draft_count(a.qo_indptr, b, a.draft_len);
  if (t >= qn) return;  // past the request's draft rows
  const size_t qrow = (size_t)(qbase + t) * a.hq + head;
  const int dcol = chunk * 64 + lane;

  // max over the splits' log-sum-exps (log2 domain)
  const size_t prow0 = (((size_t)b * a.hkv + h_kv) * a.n_splits) * a.rows + r;
  float mp = -__builtin_inff();
  for (int s = lane; s < a.n_splits; s += 64) mp = fmaxf(mp, a.part_lse[prow0 + (size_t)s * a.rows]);
  mp = wave_max(mp);

  // draft block: the draft keys row t sees (its draft-mask row, or 0..t),
  // online softmax
  float q[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) q[e] = load_elem<QDT>(a.q, qrow * D + lane + 64 * e);
  float md = -__builtin_inff();
  float ld = 0.f;
  float od = 0.f;
  const uint8_t* mrow = a.draft_mask ? a.draft_mask + ((size_t)b * a.draft_len + t) * a.draft_len : nullptr;
  const int jend = mrow ? qn : t + 1;
  for (int j = 0; j < jend; ++j) {
    if (mrow && mrow[j] == 0) continue;  // the same row for the whole wave
    const size_t krow = ((size_t)(qbase + j) * a.hkv + h_kv) * D;
    float zz = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) zz += q[e] * load_elem<KDT>(a.k_ext, krow + lane + 64 * e);
    zz = wave_sum(zz) * scale_log2_draft;
    const float mn = fmaxf(md, zz);
    const float a1 = fast_exp2(md - mn);
    const float p = fast_exp2(zz - mn);
    ld = ld * a1 + p;
    od = od * a1 + p * load_elem<KDT>(a.v_ext, krow + dcol);
    md = mn;
  }
  const float lse_d = md + fast_log2(ld);

  // merge: weights exp2(LSE_s - M); an empty split has LSE_s = -inf, O_s = 0
  const float mt = fmaxf(mp, lse_d);
  const float wd = fast_exp2(lse_d - mt);
  float wsum = wd;
  float acc = ld > 0.f ? od * (wd / ld) : 0.f;
  const float* po = a.part_o + prow0 * D + dcol;
  const size_t sstride = (size_t)a.rows * D;
  int s = 0;
  for (; s + 8 <= a.n_splits; s += 8) {
    float w[8], x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      w[u] = fast_exp2(a.part_lse[prow0 + (size_t)(s + u) * a.rows] - mt);
      x[u] = po[(size_t)(s + u) * sstride];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      wsum += w[u];
      acc += w[u] * x[u];
    }
  }
  for (; s < a.n_splits; ++s) {
    const float w = fast_exp2(a.part_lse[prow0 + (size_t)s * a.rows] - mt);
    wsum += w;
    acc += w * po[(size_t)s * sstride];
  }
  const float v = acc * (a.v_scale / wsum);
  if constexpr (QDT == DT_F32)
    reinterpret_cast<float*>(a.o)[qrow * D + dcol] = v;
  else
    reinterpret_cast<__bf16*>(a.o)[qrow * D + dcol] = (__bf16)v;
  if (lane == 0 && chunk == 0) a.lse[qrow] = (mt + fast_log2(wsum)) * kLn2;
}

// ===========================================================================
// Planner dump (test hook): one thread per workgroup slot
// ===========================================================================
__global__ void plan_dump_kernel(int mode, FlatArgs fa, PagedArgs pa, int64_t n_items,
                                 int32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_items) return;
  Item it;
  if (mode == 0) {
    it = flat_item((int32_t)(i / fa.hkv), (int32_t)(i % fa.hkv), fa.prefix_len, fa.nseg,
                   fa.seg_offsets, fa.tile_tokens);
  } else {
    it = paged_item((int32_t)i, pa.hkv, pa.n_splits, pa.split_len, pa.draft_len, pa.prefix_lens);
  }
  int32_t* o = out + i * 10;
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

// ===========================================================================
// launch wrappers
// ===========================================================================
template <int D, bool F32C>
static int launch_flat_t(const FlatArgs& a, int64_t n_blocks, hipStream_t s) {
  hipLaunchKernelGGL((flat_fwd_kernel<D, F32C>), dim3((unsigned)n_blocks), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

// fp32 inputs run flat_fwd_kernel; bf16 runs the LDS-DMA kernel of psattn_flat.hip
int launch_flat(const FlatArgs& a, int d, int dtype, int64_t n_blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype != DT_F32) return launch_flat_bf16(a, d, n_blocks, stream);
  switch (d) {
    case 64: return launch_flat_t<64, true>(a, n_blocks, s);
    case 128: return launch_flat_t<128, true>(a, n_blocks, s);
    case 256: return launch_flat_t<256, true>(a, n_blocks, s);
  }
  return (int)hipErrorInvalidValue;
}

template <int D, int KDT, int RB>
static int launch_split_t(const PagedArgs& a, int64_t n_blocks, hipStream_t s) {
  hipLaunchKernelGGL((paged_split_kernel<D, KDT, RB>), dim3((unsigned)n_blocks), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

template <int D, int KDT>
static int launch_split_rb(const PagedArgs& a, int rb, int64_t n_blocks, hipStream_t s) {
  switch (rb) {
    case 1:
      if constexpr (KDT == DT_F32 && D >= 256) return (int)hipErrorInvalidValue;
      else return launch_split_t<D, KDT, 1>(a, n_blocks, s);
    case 2: return launch_split_t<D, KDT, 2>(a, n_blocks, s);
    case 4: return launch_split_t<D, KDT, 4>(a, n_blocks, s);
  }
  return (int)hipErrorInvalidValue;
}

template <int D, int QDT, int KDT>
static int launch_combine_t(const PagedArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.batch * a.hkv * a.rows * (D / 64);
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((paged_combine_kernel<D, QDT, KDT>), dim3((unsigned)blocks), dim3(256), 0, s, a, a.scale_log2);
  return (int)hipGetLastError();
}

template <int D>
static int launch_combine_d(const PagedArgs& a, int kv_dtype, hipStream_t s) {
  if (kv_dtype == DT_F32) return launch_combine_t<D, DT_F32, DT_F32>(a, s);
  if (kv_dtype == DT_BF16) return launch_combine_t<D, DT_BF16, DT_BF16>(a, s);
  return launch_combine_t<D, DT_BF16, DT_FP8>(a, s);
}

int launch_paged_combine(const PagedArgs& a, int d, int q_dtype, int kv_dtype, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)q_dtype;  // q dtype follows kv dtype: f32 with f32, bf16 otherwise
  switch (d) {
    case 64: return launch_combine_d<64>(a, kv_dtype, s);
    case 128: return launch_combine_d<128>(a, kv_dtype, s);
    case 256: return launch_combine_d<256>(a, kv_dtype, s);
  }
  return (int)hipErrorInvalidValue;
}

template <int D>
static int launch_tiled_d(const PagedArgs& a, int kv_dtype, int rb, int64_t n_blocks, hipStream_t s) {
  if (kv_dtype == DT_F32) return launch_split_rb<D, DT_F32>(a, rb, n_blocks, s);
  if (kv_dtype == DT_BF16) return launch_split_rb<D, DT_BF16>(a, rb, n_blocks, s);
  return launch_split_rb<D, DT_FP8>(a, rb, n_blocks, s);
}

int launch_paged(const PagedArgs& a, int d, int q_dtype, int kv_dtype, const PagedGeom& geo,
                 int64_t n_blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int e;
  if (geo.stream == 2 || geo.stream == 3) {
    e = geo.stream == 2 ? launch_paged_reg(a, d, kv_dtype, n_blocks, stream)
                        : launch_paged_wide(a, d, kv_dtype, n_blocks, stream);
    if (e) return e;
    return launch_paged_merge(a, d, q_dtype, stream);
  } else if (geo.stream == 1) {
    e = launch_paged_stream(a, d, kv_dtype, geo, n_blocks, stream);
  } else {
    switch (d) {
      case 64: e = launch_tiled_d<64>(a, kv_dtype, geo.row_blocks, n_blocks, s); break;
      case 128: e = launch_tiled_d<128>(a, kv_dtype, geo.row_blocks, n_blocks, s); break;
      case 256: e = launch_tiled_d<256>(a, kv_dtype, geo.row_blocks, n_blocks, s); break;
      default: e = (int)hipErrorInvalidValue;
    }
  }
  if (e) return e;
  return launch_paged_combine(a, d, q_dtype, kv_dtype, stream);
}

int launch_plan_dump(int mode, const FlatArgs* fa, const PagedArgs* pa, int64_t n_items,
                     int32_t* items, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  FlatArgs f{};
  PagedArgs p{};
  if (fa) f = *fa;
  if (pa) p = *pa;
  const int64_t blocks = (n_items + 255) / 256;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL(plan_dump_kernel, dim3((unsigned)blocks), dim3(256), 0, s, mode, f, p, n_items, items);
  return (int)hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace psattn
