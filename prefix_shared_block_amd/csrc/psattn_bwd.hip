// psattn_bwd.hip -- gradients of the flat prefix-shared forward (bf16), gfx950.
//
// PrefixSharing PR #50 ("关键变更", key changes) builds each rollout's KV by
// copying the prefix with .copy_(), so gradients flow back through the copy
// and a stored prefix row receives the sum of its copies' gradients.  On the
// flat buffer that is the gradient of one attention under the block-causal
// visibility (prefix keys seen by every later row, a rollout's keys only by
// its own later rows), computed here without any expansion:
//
//  * bwd_pre: delta = sum_d dO O and lse2 = LSE log2(e) per (row, query
//    head); zeroes the fp32 dK / dV accumulators;
//  * bwd_dq: one forward work item per workgroup (4 waves x 32 stacked query
//    rows, the same 64-key tiles and tile order as the forward):
//      S^T = K Q^T,  P^T = exp2(S^T c - lse2),  dP^T = V dO^T,
//      dS^T = P^T (dP^T - delta),  dQ^T += K^T dS^T  (dQ = sm_scale dQ^T^T);
//  * bwd_dkdv: a tile of 128 keys of one kv head per workgroup (32 per wave,
//    their K^T and V^T fragments in registers) against one chunk of the query
//    rows that see them, streamed as tiles of 64 stacked rows (copied
//    global -> LDS three tiles ahead in a ring of four buffers):
//      S = Q K^T,  P = exp2(S c - lse2),  dP = dO V^T,  dS = P (dP - delta),
//      dV^T += dO^T P,  dK^T += Q^T dS;
//    each item adds its partial dK / dV into the fp32 accumulators (a prefix
//    key is seen by many chunks);
//  * bwd_post: dK = sm_scale acc_k and dV = acc_v, to bf16.
//
// Tiles that are read both by rows (an MFMA A operand) and transposed
// (ds_read_b64_tr_b16) keep chunk c of row r at c ^ (4 (r & 3) + (r >> 2 & 3)):
// a 16-row pass at one chunk and a 4-row x 4-chunk transposed pass then both
// touch 16 different chunk slots.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

#include <type_traits>

namespace psattn {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

#define PB_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

template <int D>
struct BCfg {
  static constexpr int ROWB = 2 * D;       // bytes of a bf16 row
  static constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
  static constexpr int NSTEP = D / 16;     // k-steps over the head dimension
  static constexpr int NDB = D / 32;       // 32-column blocks of the head dimension
  static_assert(CPR == 16, "the two-way swizzle assumes 16 chunks per row");
  // rows read both ways
  __device__ static constexpr int fb(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
  // rows read by rows only
  __device__ static constexpr int fk(int r) { return r & (CPR - 1); }
};

// ------------------------------------------------------------------- dQ pass
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int BN = 64;
  constexpr int TILE = BN * C::ROWB;
  constexpr int NCOPY = TILE / 1024;
  constexpr int CPW = 2 * NCOPY / kWaves;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // [buffer][K, V]

  const int blk = blockIdx.x;
  const int h_kv = blk % a.hkv;
  const Item it = flat_item(blk / a.hkv, h_kv, a.prefix_len, a.nseg, a.seg_offsets, a.tile_tokens);
  if (it.kind == kNone) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int r = wave * kWaveRows + l32;
  const int tok = r / a.g;
  const int hl = r - tok * a.g;
  const int token = it.q_begin + tok;
  const bool valid = (tok < a.tile_tokens) && (token < it.q_end);
  const int token_c = valid ? token : it.q_begin;
  const size_t qrow = (size_t)token_c * a.hq + h_kv * a.g + hl;

  // Q^T and dO^T fragments: k-step s, lane group g holds d = 16 s + 8 g .. +8
  bf16x8_t qf[C::NSTEP], df[C::NSTEP];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + qrow * D;
    const __bf16* dp = reinterpret_cast<const __bf16*>(a.dout) + qrow * D;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * s + 8 * g);
      df[s] = *reinterpret_cast<const bf16x8_t*>(dp + 16 * s + 8 * g);
    }
  }
  // rows outside the item weigh nothing: lse2 = +inf makes their P zero
  const float lse2 = valid ? a.lse2[qrow] : __builtin_inff();
  const float delta = valid ? a.delta[qrow] : 0.f;

  const int n0 = cdiv32(it.r0_end - it.r0_begin, BN);
  const int n1 = cdiv32(it.r1_end - it.r1_begin, BN);
  const int nt = n0 + n1;
  auto n_clean = [&](int b, int e) __attribute__((always_inline)) {
    const int whole = (e - b) / BN;
    const int causal = it.q_begin + 1 - b >= 0 ? (it.q_begin + 1 - b) / BN : 0;
    return whole < causal ? whole : causal;
  };
  const int c0 = n0 > 0 ? n_clean(it.r0_begin, it.r0_end) : 0;
  const int c1 = n1 > 0 ? n_clean(it.r1_begin, it.r1_end) : 0;
  const int nc = c0 + c1;
  auto tile_range = [&](int n, int& k0, int& ke) __attribute__((always_inline)) {
    if (n < c0) {
      k0 = it.r0_begin + n * BN;
      ke = it.r0_end;
    } else if (n < nc) {
      k0 = it.r1_begin + (n - c0) * BN;
      ke = it.r1_end;
    } else if (n < nc + n0 - c0) {
      k0 = it.r0_begin + (n - c1) * BN;
      ke = it.r0_end;
    } else {
      k0 = it.r1_begin + (n - n0) * BN;
      ke = it.r1_end;
    }
  };

  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)h_kv * C::ROWB;
  const char* vbase = reinterpret_cast<const char*>(a.v) + (size_t)h_kv * C::ROWB;
  const uint32_t row_stride = (uint32_t)a.hkv * C::ROWB;
  const bool w_isv = wave * CPW >= NCOPY;
  const char* wbase = w_isv ? vbase : kbase;
  // K is read by rows and transposed (swizzle fb), V by rows only (fk)
  auto swz = [&](int row) __attribute__((always_inline)) { return w_isv ? C::fk(row) : C::fb(row); };
  // Copy t of this wave is 1 KiB block jb = (wave CPW + t) mod NCOPY: rows
  // 4 jb .. 4 jb + 3 (the row part of the source offset goes to the scalar
  // base), lane l on row 4 jb + l / 16, chunk l % 16.  With 16 chunks per row
  // both swizzles reduce to copy 0's lane offset with bits flipped by t & 3:
  // bits 4..5 for fb (K), bits 6..7 for fk (V).
  static_assert(C::CPR == 16 && CPW % 4 == 0, "copy offsets repeat with period 4");
  const uint32_t coff0 = (uint32_t)(lane / C::CPR) * row_stride +
                         16u * (uint32_t)((lane % C::CPR) ^ swz(4 * ((wave * CPW) % NCOPY) + lane / C::CPR));
  const uint32_t cflip = w_isv ? 64u : 16u;
  auto issue = [&](int n, int bsel) __attribute__((always_inline)) {
    const uint32_t bofs = (uint32_t)bsel * (2 * TILE);
    int k0, ke;
    tile_range(n, k0, ke);
    const char* base = wbase + (size_t)k0 * row_stride;
    if (k0 + BN <= ke) {
#pragma unroll
      for (int t = 0; t < CPW; ++t) {
        const int jb = (wave * CPW + t) % NCOPY;
        dma16_s(base + (size_t)(4 * jb) * row_stride, coff0 ^ (cflip * (uint32_t)(t & 3)),
                lds_addr(&smem[0][w_isv ? 1 : 0][jb * 1024]) + bofs);
      }
    } else {
      const int lastr = ke - 1 - k0;
#pragma unroll
      for (int t = 0; t < CPW; ++t) {
        const int jb = (wave * CPW + t) % NCOPY;
        const int p = jb * 64 + lane;
        const int row = p / C::CPR;
        const int pos = p % C::CPR;
        const int rc = row < lastr ? row : lastr;
        const uint32_t off = (uint32_t)rc * row_stride + 16u * (uint32_t)(pos ^ swz(row));
        dma16_s(base, off, lds_addr(&smem[0][w_isv ? 1 : 0][jb * 1024]) + bofs);
      }
    }
  };

  f32x16_t dq[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
  const float c = a.scale_log2;
  const int li = lane & 15;
  const int sp = li >> 2;
  const int ap = li & 3;
  const int hgrp = l32 >> 4;

  auto math = [&](const char* kt, const char* vt, int key0, int kend, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    // lane (l32, g), reg i of block kb: key 32 kb + 8 (i / 4) + 4 g + i % 4 of row l32
    int lim = BN;
    if constexpr (MASK) lim = (kend < token + 1 ? kend : token + 1) - key0;
    bf16x8_t dst[4];  // k-step ks = 2 kb + half: regs 8 half .. 8 half + 7 of block kb
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t sc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sc[e] = 0.f;
        dp[e] = 0.f;
      }
      const int row = 32 * kb + l32;
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + row * C::ROWB + 16 * ((2 * s + g) ^ C::fb(row)));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(vt + row * C::ROWB + 16 * ((2 * s + g) ^ C::fk(row)));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[s], dp, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(__builtin_fmaf(sc[i], c, -lse2));
        if constexpr (MASK) {
          const int kr = 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          p = kr < lim ? p : 0.f;
        }
        dst[2 * kb + (i >> 3)][i & 7] = (__bf16)(p * (dp[i] - delta));
      }
    }
    // dQ^T += K^T dS^T: A operand lane (d, g) = K rows 16 ks + 8 t + 4 g + 0..3
    // of column d, read transposed
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        s16x4_t vv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = 16 * ks + 8 * t + 4 * g + sp;
          const int chunk = 4 * db + 2 * hgrp + (ap >> 1);
          vv[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              PB_LDS_PTR(s16x4_t, kt + row * C::ROWB + 16 * (chunk ^ C::fb(row)) + 8 * (ap & 1)));
        }
        const s16x8_t v8 = {vv[0][0], vv[0][1], vv[0][2], vv[0][3], vv[1][0], vv[1][1], vv[1][2], vv[1][3]};
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v8), dst[ks], dq[db], 0, 0, 0);
      }
    }
  };

  auto compute = [&](int n, auto maskc) __attribute__((always_inline)) {
    int k0, ke;
    tile_range(n, k0, ke);
    math(smem[n & 1][0], smem[n & 1][1], k0, ke, maskc);
  };

  // the first tile's copies go out with the fragment loads in flight; all are
  // retired before the loop, whose copies are waited for explicitly
  if (nt > 0) issue(0, 0);
#pragma unroll
  for (int s = 0; s < C::NSTEP; ++s) asm volatile("" ::"v"(qf[s]), "v"(df[s]));
  wait_vmcnt<0>();
  __syncthreads();
  int n = 0;
  for (; n < nc; ++n) {
    if (n + 1 < nt) issue(n + 1, (n + 1) & 1);
    compute(n, std::false_type{});
    wait_vmcnt<0>();
    __syncthreads();
  }
  for (; n < nt; ++n) {
    if (n + 1 < nt) issue(n + 1, (n + 1) & 1);
    compute(n, std::true_type{});
    wait_vmcnt<0>();
    __syncthreads();
  }

  // dQ = sm_scale (dQ^T)^T: staged through LDS (chunk c of row r at
  // c ^ (r % CPR)) so that every store is a whole 16-byte chunk of a row
  const float sc_out = a.sm_scale;
  char* ost = &smem[0][0][0] + wave * (kWaveRows * C::ROWB);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x2_t v = {pack_bf16x2(dq[db][4 * g4] * sc_out, dq[db][4 * g4 + 1] * sc_out),
                         pack_bf16x2(dq[db][4 * g4 + 2] * sc_out, dq[db][4 * g4 + 3] * sc_out)};
      *reinterpret_cast<u32x2_t*>(ost + l32 * C::ROWB + 16 * ((4 * db + g4) ^ (l32 & (C::CPR - 1))) + 8 * g) = v;
    }
  }
  __syncthreads();
  constexpr int NOUT = kWaveRows * C::CPR / 64;
#pragma unroll
  for (int k = 0; k < NOUT; ++k) {
    const int p = 64 * k + lane;
    const int row = p / C::CPR;
    const int ch = p % C::CPR;
    const int rr = wave * kWaveRows + row;
    const int tk = rr / a.g;
    const int hh = rr - tk * a.g;
    const int tkn = it.q_begin + tk;
    if (tk < a.tile_tokens && tkn < it.q_end) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(ost + row * C::ROWB + 16 * (ch ^ (row & (C::CPR - 1))));
      __bf16* op = reinterpret_cast<__bf16*>(a.dq) + ((size_t)tkn * a.hq + h_kv * a.g + hh) * D + 8 * ch;
      *reinterpret_cast<u32x4_t*>(op) = x;
    }
  }
}

// --------------------------------------------------------------- dK/dV pass
template <int D>
// One wave per SIMD: the fixed K^T / V^T fragments (64 VGPRs) and the two
// accumulators (128) leave too little of a 256-register budget; at two waves
// per SIMD the spills cost more than the second wave gains.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int RT = 64;                  // stacked query rows per tile
  constexpr int TILE = RT * C::ROWB;      // Q (or dO) tile bytes
  constexpr int NCOPY = TILE / 1024;      // 1 KiB copies per Q (or dO) tile
  constexpr int CPW = 2 * NCOPY / kWaves; // copies per wave per tile
  constexpr int NBUF = 4;                                        // tile ring (NBUF - 1 tiles ahead)
  __shared__ __attribute__((aligned(1024))) char smem[NBUF][2][TILE];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float rowv[NBUF][2][RT];     // [buffer][lse2, delta]
  __shared__ __attribute__((aligned(16))) int tokoff[RT];           // token offset of stacked row s

  const int blk = blockIdx.x;
  const int h_kv = blk % a.hkv;
  const BwdItem bi = dkdv_item(blk / a.hkv, a.prefix_len, a.nseg, a.seg_offsets, a.row_chunk);
  if (!bi.valid) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int G = a.g;
  const int TT = RT / G;          // query tokens per tile
  const int vrows_full = TT * G;  // valid stacked rows of a whole tile

  if (tid < RT) tokoff[tid] = tid / G;

  // this lane's key: column l32 of the wave's 32 keys
  const int key = bi.k0 + 32 * wave + l32;
  const bool kvalid = key < bi.k1;
  const int key_c = kvalid ? key : bi.k1 - 1;
  // K^T and V^T fragments (B operands): k-step s, lane group g holds
  // d = 16 s + 8 g .. +8 of this lane's key
  bf16x8_t kf[C::NSTEP], vf[C::NSTEP];
  {
    const size_t krow = ((size_t)key_c * a.hkv + h_kv) * D;
    const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + krow;
    const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + krow;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8_t*>(kp + 16 * s + 8 * g);
      vf[s] = *reinterpret_cast<const bf16x8_t*>(vp + 16 * s + 8 * g);
    }
  }

  const int ntile = cdiv32(bi.r1 - bi.r0, TT);
  // masked tiles: those with a row token below the last key (causal), and the
  // last tile when it is partial (or when G does not divide RT); they run
  // first, then the clean ones
  const int kmax = bi.k1 - 1;  // last key of the item
  int ndiag = kmax > bi.r0 ? cdiv32(kmax - bi.r0, TT) : 0;
  ndiag = ndiag < ntile ? ndiag : ntile;
  // when G does not divide RT every tile has unused rows: all are masked
  const bool all_mask = vrows_full < RT;
  const bool extra = !all_mask && ((bi.r1 - bi.r0) % TT != 0) && ntile > ndiag;  // partial last tile
  const int nmask = all_mask ? ntile : ndiag + (extra ? 1 : 0);
  auto tile_of = [&](int n) __attribute__((always_inline)) {
    if (all_mask || n < ndiag) return n;
    if (extra) return n == ndiag ? ntile - 1 : n - 1;
    return n;
  };

  // copies: waves 0, 1 copy the Q tile, waves 2, 3 the dO tile; copy t of a
  // wave is 1 KiB block jb, lane l on stacked row s = 4 jb + l / 16, chunk l % 16
  const bool w_isd = wave * CPW >= NCOPY;
  const char* src = reinterpret_cast<const char*>(w_isd ? a.dout : a.q);
  const uint32_t tok_stride = (uint32_t)a.hq * C::ROWB;
  uint32_t coff[CPW];
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int jb = (wave * CPW + t) % NCOPY;
    const int s = jb * 4 + lane / C::CPR;
    const int pos = lane % C::CPR;
    const int sc_ = s < vrows_full ? s : vrows_full - 1;
    coff[t] = (uint32_t)(sc_ / G) * tok_stride + (uint32_t)(sc_ % G) * C::ROWB + 16u * (uint32_t)(pos ^ C::fb(s));
  }
  // per-row values: wave 0 copies lse2, wave 1 delta (one dword per lane)
  const float* rsrc = wave == 0 ? a.lse2 : a.delta;
  const int s_l = lane < vrows_full ? lane : vrows_full - 1;
  const uint32_t roff = (uint32_t)((s_l / G) * a.hq + (s_l % G)) * 4u;

  auto issue = [&](int n, int bsel) __attribute__((always_inline)) {
    const int tl = tile_of(n);
    const int t0 = bi.r0 + tl * TT;
    const int nv = (bi.r1 - t0 < TT ? bi.r1 - t0 : TT) * G;  // valid stacked rows
    const char* base = src + ((size_t)t0 * a.hq + (size_t)h_kv * G) * C::ROWB;
    if (nv == RT) {
#pragma unroll
      for (int t = 0; t < CPW; ++t) {
        const int jb = (wave * CPW + t) % NCOPY;
        dma16_s(base, coff[t], lds_addr(&smem[bsel][w_isd ? 1 : 0][jb * 1024]));
      }
    } else {
#pragma unroll
      for (int t = 0; t < CPW; ++t) {
        const int jb = (wave * CPW + t) % NCOPY;
        const int s = jb * 4 + lane / C::CPR;
        const int pos = lane % C::CPR;
        const int sc_ = s < nv ? s : nv - 1;
        const uint32_t off = (uint32_t)(sc_ / G) * tok_stride + (uint32_t)(sc_ % G) * C::ROWB +
                             16u * (uint32_t)(pos ^ C::fb(s));
        dma16_s(base, off, lds_addr(&smem[bsel][w_isd ? 1 : 0][jb * 1024]));
      }
    }
    if (wave < 2) {
      const float* rb = rsrc + (size_t)t0 * a.hq + (size_t)h_kv * G;
      uint32_t ro = roff;
      if (nv < RT) {
        const int sl = lane < nv ? lane : nv - 1;
        ro = (uint32_t)((sl / G) * a.hq + (sl % G)) * 4u;
      }
      dma4_s(rb, ro, lds_addr(&rowv[bsel][wave][0]));
    }
  };

  f32x16_t dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[db][e] = 0.f;
      dv[db][e] = 0.f;
    }
  const float c = a.scale_log2;
  const int li = lane & 15;
  const int sp = li >> 2;
  const int ap = li & 3;
  const int hgrp = l32 >> 4;

  auto math = [&](int bsel, int t0, int nv, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    const char* qt = smem[bsel][0];
    const char* dt = smem[bsel][1];
    const float* l2 = rowv[bsel][0];
    const float* dl = rowv[bsel][1];
#pragma unroll
    for (int rb = 0; rb < RT / 32; ++rb) {
      // lane (key l32, g), reg i: stacked row 32 rb + 8 (i / 4) + 4 g + i % 4
      f32x16_t sc, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sc[e] = 0.f;
        dp[e] = 0.f;
      }
      const int row = 32 * rb + l32;
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(qt + row * C::ROWB + 16 * ((2 * s + g) ^ C::fb(row)));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[s], sc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        const bf16x8_t da = *reinterpret_cast<const bf16x8_t*>(dt + row * C::ROWB + 16 * ((2 * s + g) ^ C::fb(row)));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[s], dp, 0, 0, 0);
      }
      bf16x8_t pb[2], db_[2];  // k-step ks (16 rows): regs 8 ks .. 8 ks + 7
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int s0 = 32 * rb + 8 * q4 + 4 * g;  // rows s0 .. s0 + 3 of regs 4 q4 .. 4 q4 + 3
        const f32x4_t lv = *reinterpret_cast<const f32x4_t*>(l2 + s0);
        const f32x4_t dv4 = *reinterpret_cast<const f32x4_t*>(dl + s0);
        int4 tv;
        if constexpr (MASK) tv = *reinterpret_cast<const int4*>(tokoff + s0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          float p = fast_exp2(__builtin_fmaf(sc[i], c, -lv[e]));
          if constexpr (MASK) {
            const int te = e == 0 ? tv.x : (e == 1 ? tv.y : (e == 2 ? tv.z : tv.w));
            const bool vis = (s0 + e < nv) && (key <= t0 + te);
            p = vis ? p : 0.f;
          }
          pb[i >> 3][i & 7] = (__bf16)p;
          db_[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dv4[e]));
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS: A operand lane (d, g) = rows
      // 32 rb + 16 ks + 8 t + 4 g + 0..3 of column d, read transposed
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int dbk = 0; dbk < C::NDB; ++dbk) {
          s16x4_t ov[2], qv[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int rr = 32 * rb + 16 * ks + 8 * t + 4 * g + sp;
            const int chunk = 4 * dbk + 2 * hgrp + (ap >> 1);
            const int off = rr * C::ROWB + 16 * (chunk ^ C::fb(rr)) + 8 * (ap & 1);
            ov[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PB_LDS_PTR(s16x4_t, dt + off));
            qv[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PB_LDS_PTR(s16x4_t, qt + off));
          }
          const s16x8_t o8 = {ov[0][0], ov[0][1], ov[0][2], ov[0][3], ov[1][0], ov[1][1], ov[1][2], ov[1][3]};
          const s16x8_t q8 = {qv[0][0], qv[0][1], qv[0][2], qv[0][3], qv[1][0], qv[1][1], qv[1][2], qv[1][3]};
          dv[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, o8), pb[ks], dv[dbk], 0, 0, 0);
          dk[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, q8), db_[ks], dk[dbk], 0, 0, 0);
        }
      }
    }
  };

  auto compute = [&](int n, int bsel, auto maskc) __attribute__((always_inline)) {
    const int tl = tile_of(n);
    const int t0 = bi.r0 + tl * TT;
    const int nv = (bi.r1 - t0 < TT ? bi.r1 - t0 : TT) * G;
    math(bsel, t0, nv, maskc);
  };

  // copies complete in issue order: CPW per tile and wave, plus the row
  // values for waves 0 and 1
  auto wait_tile = [&](int m, int last) __attribute__((always_inline)) {
    const int later = last - m;
    if (later <= 0) wait_vmcnt<0>();
    else if (wave < 2) {
      if (later == 1) wait_vmcnt<CPW + 1>(); else wait_vmcnt<2 * (CPW + 1)>();
    } else {
      if (later == 1) wait_vmcnt<CPW>(); else wait_vmcnt<2 * CPW>();
    }
  };
  const int lastp = (ntile < NBUF - 1 ? ntile : NBUF - 1) - 1;
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < ntile) issue(p, p);
#pragma unroll
  for (int s = 0; s < C::NSTEP; ++s) asm volatile("" ::"v"(kf[s]), "v"(vf[s]));
  wait_tile(0, lastp);
  __syncthreads();
  int n = 0;
  for (; n < nmask; ++n) {
    const int nx = n + NBUF - 1;
    if (nx < ntile) issue(nx, nx % NBUF);
    compute(n, n % NBUF, std::true_type{});
    wait_tile(n + 1, nx < ntile - 1 ? nx : ntile - 1);
    __syncthreads();
  }
  for (; n < ntile; ++n) {
    const int nx = n + NBUF - 1;
    if (nx < ntile) issue(nx, nx % NBUF);
    compute(n, n % NBUF, std::false_type{});
    wait_tile(n + 1, nx < ntile - 1 ? nx : ntile - 1);
    __syncthreads();
  }

  // Add the item's partial dK^T / dV^T into the fp32 accumulators.  Each wave
  // stages its [32 keys][D] block in LDS (16-byte chunk c of key row kr at
  // c ^ kr), then adds it with consecutive lanes on consecutive floats.
  constexpr int SROW = D * 4;
  static_assert(kWaves * 32 * SROW <= NBUF * 2 * TILE, "staging fits in the tiles");
  char* st = &smem[0][0][0] + wave * (32 * SROW);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int dbk = 0; dbk < C::NDB; ++dbk)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // C layout: lane (key l32, g), regs 4 q4 .. 4 q4 + 3 hold d = 32 dbk + 8 q4 + 4 g .. +3
        const f32x4_t x = which == 0 ? f32x4_t{dv[dbk][4 * q4], dv[dbk][4 * q4 + 1], dv[dbk][4 * q4 + 2], dv[dbk][4 * q4 + 3]}
                                     : f32x4_t{dk[dbk][4 * q4], dk[dbk][4 * q4 + 1], dk[dbk][4 * q4 + 2], dk[dbk][4 * q4 + 3]};
        *reinterpret_cast<f32x4_t*>(st + l32 * SROW + 16 * ((8 * dbk + 2 * q4 + g) ^ l32)) = x;
      }
    __syncthreads();
    float* acc = which == 0 ? a.acc_v : a.acc_k;
#pragma unroll 4
    for (int p = lane; p < 32 * D; p += 64) {
      const int kr = p / D;
      const int f = p % D;
      const int kk = bi.k0 + 32 * wave + kr;
      if (kk < bi.k1) {
        const float x = *reinterpret_cast<const float*>(st + kr * SROW + 16 * ((f >> 2) ^ kr) + 4 * (f & 3));
        unsafeAtomicAdd(acc + ((size_t)kk * a.hkv + h_kv) * D + f, x);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- pre and post passes
// delta and lse2 for rows [T * Hq]: 16 lanes per row (8 elements each); the
// accumulators are zeroed by the same grid
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, int64_t nrows, int64_t nacc4) {
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gtid / (D / 8);
  const int part = (int)(gtid % (D / 8));
  float s = 0.f;
  if (row < nrows) {
    const u32x4_t o4 = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const __bf16*>(a.o) + row * D + 8 * part);
    const u32x4_t d4 = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const __bf16*>(a.dout) + row * D + 8 * part);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float o0 = __builtin_bit_cast(float, o4[w] << 16), o1 = __builtin_bit_cast(float, o4[w] & 0xffff0000u);
      const float d0 = __builtin_bit_cast(float, d4[w] << 16), d1 = __builtin_bit_cast(float, d4[w] & 0xffff0000u);
      s = __builtin_fmaf(o0, d0, s);
      s = __builtin_fmaf(o1, d1, s);
    }
  }
#pragma unroll
  for (int m = 1; m < D / 8; m <<= 1) s += __shfl_xor(s, m);
  if (row < nrows && part == 0) {
    a.delta[row] = s;
    a.lse2[row] = a.lse[row] * kLog2e;
  }
  const int64_t nthr = (int64_t)gridDim.x * 256;
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = gtid; i < nacc4; i += nthr) {
    reinterpret_cast<f32x4_t*>(a.acc_k)[i] = z;
    reinterpret_cast<f32x4_t*>(a.acc_v)[i] = z;
  }
}

// dK = sm_scale acc_k, dV = acc_v, 8 elements per thread
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdArgs a, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4_t* k4 = reinterpret_cast<const f32x4_t*>(a.acc_k) + 2 * i;
  const f32x4_t* v4 = reinterpret_cast<const f32x4_t*>(a.acc_v) + 2 * i;
  const f32x4_t ka = k4[0], kb = k4[1], va = v4[0], vb = v4[1];
  const float s = a.sm_scale;
  const u32x4_t ko = {pack_bf16x2(ka[0] * s, ka[1] * s), pack_bf16x2(ka[2] * s, ka[3] * s),
                      pack_bf16x2(kb[0] * s, kb[1] * s), pack_bf16x2(kb[2] * s, kb[3] * s)};
  const u32x4_t vo = {pack_bf16x2(va[0], va[1]), pack_bf16x2(va[2], va[3]), pack_bf16x2(vb[0], vb[1]),
                      pack_bf16x2(vb[2], vb[3])};
  reinterpret_cast<u32x4_t*>(a.dk)[i] = ko;
  reinterpret_cast<u32x4_t*>(a.dv)[i] = vo;
}

template <int D>
int launch_bwd_t(const BwdArgs& a, int64_t dq_blocks, int64_t dkdv_blocks, hipStream_t s) {
  const int64_t nrows = a.total_tokens * a.hq;
  const int64_t nacc4 = a.total_tokens * a.hkv * D / 4;
  const int64_t pre_threads = nrows * (D / 8);
  int64_t pre_blocks = (pre_threads + 255) / 256;
  if (pre_blocks < 1) pre_blocks = 1;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_blocks), dim3(256), 0, s, a, nrows, nacc4);
  int err = (int)hipGetLastError();
  if (err) return err;
  if (dq_blocks > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)dq_blocks), dim3(kThreads), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
  }
  if (dkdv_blocks > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)dkdv_blocks), dim3(kThreads), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
  }
  const int64_t n8 = a.total_tokens * a.hkv * D / 8;
  if (n8 > 0) {
    hipLaunchKernelGGL(bwd_post_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, n8);
    if ((err = (int)hipGetLastError())) return err;
  }
  return 0;
}

}  // namespace

int launch_flat_bwd(const BwdArgs& a, int d, int64_t dq_blocks, int64_t dkdv_blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d == 128) return launch_bwd_t<128>(a, dq_blocks, dkdv_blocks, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace psattn
