// psattn_bwd.hip -- gradients of the flat prefix-shared forward (bf16), gfx950.
//
// PrefixSharing PR #50 ("关键变更", key changes) builds each rollout's KV by
// copying the prefix with .copy_(), so gradients flow back through the copy
// and a stored prefix row receives the sum of its copies' gradients.  On the
// flat buffer that is the gradient of one attention under the block-causal
// visibility (prefix keys seen by every later row, a rollout's keys only by
// its own later rows), computed here without any expansion:
//
//  * bwd_dq: one forward work item per workgroup (4 waves x 32 stacked query
//    rows, the same 64-key tiles and tile order as the forward); it also
//    forms its rows' delta = sum_d dO O and lse2 = LSE log2(e), zeroes the
//    fp32 dK / dV accumulators and writes the dK/dV item table:
//      S^T = K Q^T,  P^T = exp2(S^T c - lse2),  dP^T = V dO^T,
//      dS^T = P^T (dP^T - delta),  dQ^T += K^T dS^T  (dQ = sm_scale dQ^T^T);
//  * bwd_dkdv2 (D up to 128) / bwd_dkdv (D = 256): a tile of 128 keys of one
//    kv head per workgroup against one chunk of the query rows that see them,
//    streamed as tiles of 64 stacked rows (copied global -> LDS, one tile
//    ahead):
//      S = Q K^T,  P = exp2(S c - lse2),  dP = dO V^T,  dS = P (dP - delta),
//      dV^T += dO^T P,  dK^T += Q^T dS;
//    bwd_dkdv2 keeps the keys' K and V rows in LDS, eight waves (two per
//    SIMD) in pairs over 32 keys, each wave one 32-row block of every tile;
//    bwd_dkdv keeps a wave's 32 keys' fragments in registers, one wave per
//    SIMD, in two 128-column passes.  Each item adds its partial dK / dV into
//    the fp32 accumulators (a prefix key is seen by many chunks);
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

// a pointer every lane holds the same value of, as a scalar
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

template <int D>
struct BCfg {
  static constexpr int ROWB = 2 * D;       // bytes of a bf16 row
  static constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
  static constexpr int RPK = 1024 / ROWB;  // rows per 1 KiB copy block
  static constexpr int NSTEP = D / 16;     // k-steps over the head dimension
  static constexpr int NDB = D / 32;       // 32-column blocks of the head dimension
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "head dims 64, 128 and 256");
  // Rows read both ways.  256-byte rows (D = 128): c ^ (4 (r & 3) + (r >> 2 & 3))
  // as described above; 512-byte rows (D = 256) the same (the slot moves
  // inside its 256-byte half).  128-byte rows (D = 64) put two rows in one
  // 256-byte bank row, so (row parity, slot) must differ across a pass: slot
  // c ^ (2 (r >> 1 & 3) + (r >> 3 & 1)) does it for the 16-row pass and for the
  // 4-row x 4-half-chunk transposed pass (all checked exhaustively on the host).
  __device__ static constexpr int fb(int r) {
    return CPR != 8 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
  }
  // rows read by rows only (with 128-byte rows, by the row pair)
  __device__ static constexpr int fk(int r) { return CPR != 8 ? (r & 15) : ((r >> 1) & 7); }
};

// ------------------------------------------------------------------- dQ pass
// CHAIN: multi-level sharing (seg_parent set): after the item's own walk
// (the prefix, then its rollout up to its tile), one pass per ancestor
// segment walks that segment's keys, all visible (the forward's walk).
// One wave per SIMD at D = 256 (its Q^T and dO^T fragments and dQ^T
// accumulators alone take 256 registers), two below.
template <int D, bool CHAIN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
void bwd_dq_kernel(BwdArgs a) {
  using C = BCfg<D>;
  constexpr int BN = 64;
  constexpr int TILE = BN * C::ROWB;
  constexpr int NCOPY = TILE / 1024;
  constexpr int CPW = 2 * NCOPY / kWaves;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // [buffer][K, V]

  const int blk = blockIdx.x;
  // The launch's other duties, whatever the workgroup's item: zero the fp32
  // dK / dV accumulators and write the key-major pass's item table (entry j:
  // item j of a kv head; entry n_tab: the first item past the one-item
  // launch), both read only by the later dK/dV launches.
  // (workgroup-uniform loop bounds, so that control flow reconverges at
  // every step and the copies' base addresses stay scalar below)
  {
    const int64_t nthr = (int64_t)gridDim.x * kThreads;
    const int64_t g0 = (int64_t)blk * kThreads;
    const int64_t nacc4 = (int64_t)a.total_tokens * a.hkv * (D / 4);
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i0 = g0; i0 < nacc4; i0 += nthr) {
      const int64_t i = i0 + threadIdx.x;
      if (i < nacc4) {
        reinterpret_cast<f32x4_t*>(a.acc_k)[i] = z;
        reinterpret_cast<f32x4_t*>(a.acc_v)[i] = z;
      }
    }
    for (int64_t j0 = g0; j0 <= a.n_tab; j0 += nthr) {
      const int64_t j = j0 + threadIdx.x;
      if (j <= a.n_tab) {
        const BwdItem bi = dkdv_item((int32_t)j, a.prefix_len, a.nseg, a.seg_offsets, a.seg_parent, a.row_chunk);
        const int4 e = bi.valid ? int4{bi.k0, bi.k1, bi.r0, bi.r1} : int4{0, 0, 0, 0};
        *reinterpret_cast<int4*>(a.item_tab + 4 * j) = e;
      }
    }
  }
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
  // The row terms, formed here for the item's rows (every query row belongs
  // to exactly one dQ item) and written for the key-major pass:
  // delta = sum_d dO O (this lane's dims, then the row's other lane group)
  // and lse2 = LSE log2 e.  Rows outside the item weigh nothing: lse2 = +inf
  // makes their P zero.
  float delta = 0.f;
  if (valid) {
    const __bf16* op = reinterpret_cast<const __bf16*>(a.o) + qrow * D;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) {
      const bf16x8_t ov = *reinterpret_cast<const bf16x8_t*>(op + 16 * s + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) delta = __builtin_fmaf((float)ov[e], (float)df[s][e], delta);
    }
  }
  delta += __shfl_xor(delta, 32);
  const float lse2 = valid ? a.lse[qrow] * kLog2e : __builtin_inff();
  if (valid && g == 0) {
    a.delta[qrow] = delta;
    a.lse2[qrow] = lse2;
  }

  // key ranges of the current pass (CHAIN: later passes put an ancestor
  // segment's range in r0, all of it at or before the item's first row)
  int r0b = it.r0_begin, r0e = it.r0_end, r1b = it.r1_begin, r1e = it.r1_end;
  int n0 = cdiv32(r0e - r0b, BN);
  int n1 = cdiv32(r1e - r1b, BN);
  int nt = n0 + n1;
  auto n_clean = [&](int b, int e) __attribute__((always_inline)) {
    const int whole = (e - b) / BN;
    const int causal = it.q_begin + 1 - b >= 0 ? (it.q_begin + 1 - b) / BN : 0;
    return whole < causal ? whole : causal;
  };
  int c0 = n0 > 0 ? n_clean(r0b, r0e) : 0;
  int c1 = n1 > 0 ? n_clean(r1b, r1e) : 0;
  int nc = c0 + c1;
  auto tile_range = [&](int n, int& k0, int& ke) __attribute__((always_inline)) {
    if (n < c0) {
      k0 = r0b + n * BN;
      ke = r0e;
    } else if (n < nc) {
      k0 = r1b + (n - c0) * BN;
      ke = r1e;
    } else if (n < nc + n0 - c0) {
      k0 = r0b + (n - c1) * BN;
      ke = r0e;
    } else {
      k0 = r1b + (n - n0) * BN;
      ke = r1e;
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
  // RPK jb .. RPK jb + RPK - 1 (the row part of the source offset goes to the
  // scalar base), lane l on row RPK jb + l / CPR, chunk l % CPR.  With 16
  // chunks per row both swizzles reduce to copy 0's lane offset with bits
  // flipped by t & 3: bits 4..5 for fb (K), bits 6..7 for fk (V); with 8,
  // each copy keeps its own offset.
  static_assert(C::CPR != 16 || CPW % 4 == 0, "copy offsets repeat with period 4");
  const uint32_t coff0 = (uint32_t)(lane / C::CPR) * row_stride +
                         16u * (uint32_t)((lane % C::CPR) ^ swz(C::RPK * ((wave * CPW) % NCOPY) + lane / C::CPR));
  const uint32_t cflip = w_isv ? 64u : 16u;
  uint32_t coffs[C::CPR == 16 ? 1 : CPW];
  if constexpr (C::CPR != 16) {
#pragma unroll
    for (int t = 0; t < CPW; ++t) {
      const int jb = (wave * CPW + t) % NCOPY;
      coffs[t] = (uint32_t)(lane / C::CPR) * row_stride +
                 16u * (uint32_t)((lane % C::CPR) ^ swz(C::RPK * jb + lane / C::CPR));
    }
  }
  auto issue = [&](int n, int bsel) __attribute__((always_inline)) {
    const uint32_t bofs = (uint32_t)bsel * (2 * TILE);
    int k0, ke;
    tile_range(n, k0, ke);
    const char* base = wbase + (size_t)k0 * row_stride;
    if (k0 + BN <= ke) {
#pragma unroll
      for (int t = 0; t < CPW; ++t) {
        const int jb = (wave * CPW + t) % NCOPY;
        const uint32_t off = C::CPR == 16 ? coff0 ^ (cflip * (uint32_t)(t & 3)) : coffs[C::CPR == 16 ? 0 : t];
        dma16_s(base + (size_t)(C::RPK * jb) * row_stride, off, lds_addr(&smem[0][w_isv ? 1 : 0][jb * 1024]) + bofs);
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
  int anc = CHAIN && it.kind == kFlatSuffix && a.seg_parent ? a.seg_parent[it.seg] : -1;
  int child = it.seg;
  for (;;) {
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
    if constexpr (!CHAIN) {
      break;
    } else {
      // the next ancestor segment.  A parent precedes its child and -1 is
      // the prefix, already walked; an entry outside [-1, child) ends the
      // walk, so the loop always ends and never reads outside seg_offsets.
      anc = __builtin_amdgcn_readfirstlane(anc);
      if (anc < 0 || anc >= child) break;
      child = anc;
      r0b = __builtin_amdgcn_readfirstlane(a.seg_offsets[anc]);
      r0e = __builtin_amdgcn_readfirstlane(a.seg_offsets[anc + 1]);
      r1b = r1e = 0;
      anc = a.seg_parent[anc];
      n0 = cdiv32(r0e - r0b, BN);
      n1 = 0;
      nt = n0;
      c0 = n0 > 0 ? n_clean(r0b, r0e) : 0;
      c1 = 0;
      nc = c0;
      if (nt > 0) issue(0, 0);
    }
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

// ------------------------------------------------------ dK/dV pass, D = 256
// (D up to 128 runs the two-wave kernel further below.)  One wave per SIMD,
// each holding its 32 keys' full K^T / V^T fragments in registers: at
// D = 256 the key rows would not fit in LDS beside the query tiles.
//
// The workgroup takes item first_item + blockIdx / Hkv of its kv head.
// WALK = true: it then walks on with a stride of the grid's workgroups per kv
// head, until the first item past the end (items are numbered without
// gaps).  The host sizes the one-item launch (WALK = false) from its bound on
// the rollout lengths and adds a small walking launch from the first item
// past that bound, so the result never depends on the bound.  (For WALK =
// false the loop below ends after its first pass and compiles to the
// straight-line kernel; a loop taken by every workgroup changed the schedule
// of the tile loop and cost about 9% per call.)
//
// DO: head-dim columns of dK / dV one launch accumulates, from column dofs
// (two launches of 128 columns each, S and dP formed in both, so that the
// fragments of the full row and two 128-column accumulators fit one wave's
// registers).
template <int D, int DO, bool WALK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdArgs a, int first_item, int dofs) {
  using C = BCfg<D>;
  constexpr int NDO = DO / 32;  // 32-column blocks of the accumulated columns
  const int dcol = DO == D ? 0 : dofs;  // first accumulated column (a constant when one launch covers all)
  constexpr int RT = 64;                  // stacked query rows per tile
  constexpr int TILE = RT * C::ROWB;      // Q (or dO) tile bytes
  constexpr int NCOPY = TILE / 1024;      // 1 KiB copies per Q (or dO) tile
  constexpr int CPW = 2 * NCOPY / kWaves; // copies per wave per tile
  constexpr int NBUF = D >= 256 ? 2 : 4;  // tile ring (NBUF - 1 tiles ahead; 32 KiB tiles at D = 256)
  __shared__ __attribute__((aligned(1024))) char smem[NBUF][2][TILE];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float rowv[NBUF][2][RT];     // [buffer][lse2, delta]
  __shared__ __attribute__((aligned(16))) int tokoff[RT];           // token offset of stacked row s

  const int blk = blockIdx.x;
  const int h_kv = blk % a.hkv;
  const int nper = (int)(gridDim.x / (unsigned)a.hkv);
  if constexpr (WALK) {
    // the row-terms pass left the first item past the table in entry n_tab:
    // when it is none (the host's bound held), no walking workgroup has work,
    // and one load spares each of them the enumeration
    const int4 e = *reinterpret_cast<const int4*>(a.item_tab + 4 * (size_t)a.n_tab);
    if (!(e.y > e.x)) return;
  }
  for (int item = first_item + blk / a.hkv;; item += nper) {
    // the one-item launch reads its item from the table the row-terms pass
    // wrote (one load instead of a scan over the segments, which for a
    // segment tree took longer than many items' own work); the walking
    // launch, past the table, enumerates
    BwdItem bi;
    if constexpr (!WALK) {
      const int4 e = *reinterpret_cast<const int4*>(a.item_tab + 4 * (size_t)item);
      bi = BwdItem{e.y > e.x ? 1 : 0, e.x, e.y, e.z, e.w};
    } else {
      bi = dkdv_item(item, a.prefix_len, a.nseg, a.seg_offsets, a.seg_parent, a.row_chunk);
    }
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
    // wave is 1 KiB block jb, lane l on stacked row s = RPK jb + l / CPR, chunk l % CPR
    const bool w_isd = wave * CPW >= NCOPY;
    const char* src = reinterpret_cast<const char*>(w_isd ? a.dout : a.q);
    const uint32_t tok_stride = (uint32_t)a.hq * C::ROWB;
    uint32_t coff[CPW];
  #pragma unroll
    for (int t = 0; t < CPW; ++t) {
      const int jb = (wave * CPW + t) % NCOPY;
      const int s = jb * C::RPK + lane / C::CPR;
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
      // (at D = 256 the walking variant's loop hides the base's uniformity
      // from the compiler, which then cannot give the copies a scalar base)
      if constexpr (D >= 256) base = uniform_ptr(base);
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
          const int s = jb * C::RPK + lane / C::CPR;
          const int pos = lane % C::CPR;
          const int sc_ = s < nv ? s : nv - 1;
          const uint32_t off = (uint32_t)(sc_ / G) * tok_stride + (uint32_t)(sc_ % G) * C::ROWB +
                               16u * (uint32_t)(pos ^ C::fb(s));
          dma16_s(base, off, lds_addr(&smem[bsel][w_isd ? 1 : 0][jb * 1024]));
        }
      }
      if (wave < 2) {
        const float* rb = rsrc + (size_t)t0 * a.hq + (size_t)h_kv * G;
        if constexpr (D >= 256) rb = uniform_ptr(rb);
        uint32_t ro = roff;
        if (nv < RT) {
          const int sl = lane < nv ? lane : nv - 1;
          ro = (uint32_t)((sl / G) * a.hq + (sl % G)) * 4u;
        }
        dma4_s(rb, ro, lds_addr(&rowv[bsel][wave][0]));
      }
    };

    f32x16_t dk[NDO], dv[NDO];
  #pragma unroll
    for (int db = 0; db < NDO; ++db)
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

    // One 32-row block rb of the tile: S and dP products, softmax terms, then
    // the dV / dK updates.
    auto sdp = [&](const char* qt, const char* dt, int rb, f32x16_t& sc, f32x16_t& dp) __attribute__((always_inline)) {
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
    };
    // lane (key l32, g), reg i: stacked row 32 rb + 8 (i / 4) + 4 g + i % 4
    auto soft = [&](const float* l2, const float* dl, int rb, int t0, int nv, const f32x16_t& sc, const f32x16_t& dp,
                    bf16x8_t (&pb)[2], bf16x8_t (&db_)[2], auto maskc) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(maskc)::value;
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
    };
    // dV^T += dO^T P and dK^T += Q^T dS: A operand lane (d, g) = rows
    // 32 rb + 16 ks + 8 t + 4 g + 0..3 of column d, read transposed
    auto upd = [&](const char* qt, const char* dt, int rb, const bf16x8_t (&pb)[2], const bf16x8_t (&db_)[2])
        __attribute__((always_inline)) {
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
  #pragma unroll
        for (int dbk = 0; dbk < NDO; ++dbk) {
          s16x4_t ov[2], qv[2];
  #pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int rr = 32 * rb + 16 * ks + 8 * t + 4 * g + sp;
            const int chunk = 4 * (dbk + dcol / 32) + 2 * hgrp + (ap >> 1);
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
    };
    static_assert(RT == 64, "two 32-row blocks per tile");
    auto math = [&](int bsel, int t0, int nv, auto maskc) __attribute__((always_inline)) {
      const char* qt = smem[bsel][0];
      const char* dt = smem[bsel][1];
      const float* l2 = rowv[bsel][0];
      const float* dl = rowv[bsel][1];
      f32x16_t sc0, dp0, sc1, dp1;
      bf16x8_t pb0[2], db0[2], pb1[2], db1[2];
      // one block after the other: at D = 256 a second block's scores would not
      // fit beside the key fragments
      sdp(qt, dt, 0, sc0, dp0);
      soft(l2, dl, 0, t0, nv, sc0, dp0, pb0, db0, maskc);
      upd(qt, dt, 0, pb0, db0);
      sdp(qt, dt, 1, sc1, dp1);
      soft(l2, dl, 1, t0, nv, sc1, dp1, pb1, db1, maskc);
      upd(qt, dt, 1, pb1, db1);
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
    // stages its two [32 keys][DO] blocks in LDS (16-byte chunk c of key row kr
    // at c ^ (kr mod the row's chunks)), then adds them with consecutive lanes
    // on consecutive floats.  The staging areas are the wave's own (the tile
    // loop's last barrier has retired every read of the ring), so no barrier
    // is needed; the adds run a fixed count with no branch, so that their LDS
    // reads issue in batches: a key row past the item's end adds 0 to the
    // item's last key (the accumulators start at +0 and never hold -0, so the
    // add changes nothing).  A per-lane test around each add had serialised
    // one LDS round trip per add (about 10 us per item).
    constexpr int SROW = DO * 4;
    constexpr int SMASK = SROW / 16 - 1;
    static_assert(2 * kWaves * 32 * SROW <= NBUF * 2 * TILE, "staging fits in the tiles");
    char* const st_v = &smem[0][0][0] + wave * (32 * SROW);
    char* const st_k = st_v + kWaves * (32 * SROW);
  #pragma unroll
    for (int dbk = 0; dbk < NDO; ++dbk)
  #pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // C layout: lane (key l32, g), regs 4 q4 .. 4 q4 + 3 hold d = 32 dbk + 8 q4 + 4 g .. +3
        const int off = l32 * SROW + 16 * ((8 * dbk + 2 * q4 + g) ^ (l32 & SMASK));
        *reinterpret_cast<f32x4_t*>(st_v + off) =
            f32x4_t{dv[dbk][4 * q4], dv[dbk][4 * q4 + 1], dv[dbk][4 * q4 + 2], dv[dbk][4 * q4 + 3]};
        *reinterpret_cast<f32x4_t*>(st_k + off) =
            f32x4_t{dk[dbk][4 * q4], dk[dbk][4 * q4 + 1], dk[dbk][4 * q4 + 2], dk[dbk][4 * q4 + 3]};
      }
    {
      const int kbase = bi.k0 + 32 * wave;
  #pragma unroll
      for (int which = 0; which < 2; ++which) {
        const char* stw = which == 0 ? st_v : st_k;
        float* acc = which == 0 ? a.acc_v : a.acc_k;
        // batches of 8: the reads first (the compiler keeps memory operations
        // in order around an atomic, so they are written ahead of the adds)
        constexpr int NI = 32 * DO / 64;
        static_assert(NI % 8 == 0, "batches of 8");
  #pragma unroll 1
        for (int i0 = 0; i0 < NI; i0 += 8) {
          float x[8];
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int p = lane + 64 * (i0 + j);
            const int kr = p / DO;
            const int f = p % DO;
            x[j] = *reinterpret_cast<const float*>(stw + kr * SROW + 16 * ((f >> 2) ^ (kr & SMASK)) + 4 * (f & 3));
          }
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int p = lane + 64 * (i0 + j);
            const int kr = p / DO;
            const int f = p % DO;
            const int kk = kbase + kr;
            const bool ok = kk < bi.k1;
            const int kc = ok ? kk : bi.k1 - 1;
            unsafeAtomicAdd(acc + ((size_t)kc * a.hkv + h_kv) * D + dcol + f, ok ? x[j] : 0.f);
          }
        }
      }
    }
    // the walking launch's next item refills the ring the staging areas lie in
    if constexpr (WALK) __syncthreads();
    if constexpr (!WALK) return;
  }  // items
}

// ------------------------------------------------- dK/dV pass, two waves per SIMD
constexpr int kWaves2 = 8;
constexpr int kThreads2 = 64 * kWaves2;

// For D up to 128.  Eight waves share the item's 128 keys in pairs: waves w
// and w + 4 take keys 32 (w % 4) .. +31, and each takes one 32-row block of
// every 64-row tile (w / 4).  The keys' K and V rows sit in LDS for the whole
// item (read as the B operands of the S and dP products, in the same swizzle
// as the Q / dO rows), so that a wave's registers hold only its accumulators
// and the tile's terms: two waves fit each SIMD, and one wave's softmax and
// LDS waits overlap the other's matrix work.  The Q / dO tiles are
// double-buffered (the key rows take the LDS a deeper ring would use).  At
// the end the pair's two partial sums are added in LDS and then into the fp32
// accumulators.
template <int D, bool WALK>
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv2_kernel(BwdArgs a, int first_item) {
  using C = BCfg<D>;
  static_assert(D <= 128, "two waves per SIMD up to D = 128");
  constexpr int NDO = D / 32;
  constexpr int RT = 64;                   // stacked query rows per tile
  constexpr int TILE = RT * C::ROWB;       // Q (or dO) tile bytes
  constexpr int NCOPY = TILE / 1024;       // 1 KiB copies per Q (or dO) tile
  constexpr int CPW = 2 * NCOPY / kWaves2; // tile copies per wave
  constexpr int KVB = 128 * C::ROWB;       // the item's K (or V) rows
  constexpr int KCPW = 2 * (KVB / 1024) / kWaves2;  // key-row copies per wave
  // one array: [K, V][key row], then [buffer][Q, dO] tiles; at the end the
  // eight waves' staged partial sums span both
  __shared__ __attribute__((aligned(1024))) char lds_all[2 * KVB + 2 * 2 * TILE];
  char (*const kvs)[KVB] = reinterpret_cast<char (*)[KVB]>(lds_all);
  char (*const smem)[2][TILE] = reinterpret_cast<char (*)[2][TILE]>(lds_all + 2 * KVB);
  __shared__ __attribute__((aligned(16))) float rowv[2][2][RT];      // [buffer][lse2, delta]
  __shared__ __attribute__((aligned(16))) int tokoff[RT];            // token offset of stacked row s

  const int blk = blockIdx.x;
  const int h_kv = blk % a.hkv;
  const int nper = (int)(gridDim.x / (unsigned)a.hkv);
  if constexpr (WALK) {
    const int4 e = *reinterpret_cast<const int4*>(a.item_tab + 4 * (size_t)a.n_tab);
    if (!(e.y > e.x)) return;
  }
  for (int item = first_item + blk / a.hkv;; item += nper) {
    BwdItem bi;
    if constexpr (!WALK) {
      const int4 e = *reinterpret_cast<const int4*>(a.item_tab + 4 * (size_t)item);
      bi = BwdItem{e.y > e.x ? 1 : 0, e.x, e.y, e.z, e.w};
    } else {
      bi = dkdv_item(item, a.prefix_len, a.nseg, a.seg_offsets, a.seg_parent, a.row_chunk);
    }
    if (!bi.valid) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int kw = wave & 3;   // the pair's 32 keys
    const int rb = wave >> 2;  // the wave's 32-row block of each tile
    const int G = a.g;
    const int TT = RT / G;
    const int vrows_full = TT * G;

    if (tid < RT) tokoff[tid] = tid / G;

    const int krow = 32 * kw + l32;  // this lane's key row in kvs
    const int key = bi.k0 + krow;

    // the item's key rows (rows past its end repeat its last key: finite, and
    // their columns of S never reach a result)
    {
      const uint32_t krs = (uint32_t)a.hkv * C::ROWB;
  #pragma unroll
      for (int t = 0; t < KCPW; ++t) {
        const int jb = wave * KCPW + t;                 // 1 KiB block of K (first half) or V
        const int which = jb / (KVB / 1024);
        const int jl = jb % (KVB / 1024);
        const int s = jl * C::RPK + lane / C::CPR;      // key row
        const int pos = lane % C::CPR;
        const int kr = bi.k0 + s < bi.k1 ? s : bi.k1 - 1 - bi.k0;  // row offset from the item's first key
        const char* base = reinterpret_cast<const char*>(which == 0 ? a.k : a.v) +
                           ((size_t)bi.k0 * a.hkv + h_kv) * C::ROWB;
        dma16_s(uniform_ptr(base), (uint32_t)kr * krs + 16u * (uint32_t)(pos ^ C::fb(s)),
                lds_addr(&kvs[which][jl * 1024]));
      }
    }

    const int ntile = cdiv32(bi.r1 - bi.r0, TT);
    const int kmax = bi.k1 - 1;
    int ndiag = kmax > bi.r0 ? cdiv32(kmax - bi.r0, TT) : 0;
    ndiag = ndiag < ntile ? ndiag : ntile;
    const bool all_mask = vrows_full < RT;
    const bool extra = !all_mask && ((bi.r1 - bi.r0) % TT != 0) && ntile > ndiag;
    const int nmask = all_mask ? ntile : ndiag + (extra ? 1 : 0);
    auto tile_of = [&](int n) __attribute__((always_inline)) {
      if (all_mask || n < ndiag) return n;
      if (extra) return n == ndiag ? ntile - 1 : n - 1;
      return n;
    };

    // tile copies: waves 0..3 the Q tile, 4..7 the dO tile
    const bool w_isd = wave * CPW >= NCOPY;
    const char* src = reinterpret_cast<const char*>(w_isd ? a.dout : a.q);
    const uint32_t tok_stride = (uint32_t)a.hq * C::ROWB;
    uint32_t coff[CPW];
  #pragma unroll
    for (int t = 0; t < CPW; ++t) {
      const int jb = (wave * CPW + t) % NCOPY;
      const int s = jb * C::RPK + lane / C::CPR;
      const int pos = lane % C::CPR;
      const int sc_ = s < vrows_full ? s : vrows_full - 1;
      coff[t] = (uint32_t)(sc_ / G) * tok_stride + (uint32_t)(sc_ % G) * C::ROWB + 16u * (uint32_t)(pos ^ C::fb(s));
    }
    const float* rsrc = wave == 0 ? a.lse2 : a.delta;
    const int s_l = lane < vrows_full ? lane : vrows_full - 1;
    const uint32_t roff = (uint32_t)((s_l / G) * a.hq + (s_l % G)) * 4u;

    auto issue = [&](int n, int bsel) __attribute__((always_inline)) {
      const int tl = tile_of(n);
      const int t0 = bi.r0 + tl * TT;
      const int nv = (bi.r1 - t0 < TT ? bi.r1 - t0 : TT) * G;
      const char* base = uniform_ptr(src + ((size_t)t0 * a.hq + (size_t)h_kv * G) * C::ROWB);
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
          const int s = jb * C::RPK + lane / C::CPR;
          const int pos = lane % C::CPR;
          const int sc_ = s < nv ? s : nv - 1;
          const uint32_t off = (uint32_t)(sc_ / G) * tok_stride + (uint32_t)(sc_ % G) * C::ROWB +
                               16u * (uint32_t)(pos ^ C::fb(s));
          dma16_s(base, off, lds_addr(&smem[bsel][w_isd ? 1 : 0][jb * 1024]));
        }
      }
      if (wave < 2) {
        const float* rbp = uniform_ptr(rsrc + (size_t)t0 * a.hq + (size_t)h_kv * G);
        uint32_t ro = roff;
        if (nv < RT) {
          const int sl = lane < nv ? lane : nv - 1;
          ro = (uint32_t)((sl / G) * a.hq + (sl % G)) * 4u;
        }
        dma4_s(rbp, ro, lds_addr(&rowv[bsel][wave][0]));
      }
    };

    f32x16_t dk[NDO], dv[NDO];
  #pragma unroll
    for (int db = 0; db < NDO; ++db)
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
    const char* kt = kvs[0];
    const char* vt = kvs[1];

    // the wave's block of one tile: S = Q K^T and dP = dO V^T (lane: key l32,
    // reg i: stacked row 32 rb + 8 (i / 4) + 4 g + i % 4), the softmax terms,
    // then dV^T += dO^T P and dK^T += Q^T dS over the block's 32 rows
    auto math = [&](int bsel, int t0, int nv, auto maskc) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(maskc)::value;
      const char* qt = smem[bsel][0];
      const char* dt = smem[bsel][1];
      const float* l2 = rowv[bsel][0];
      const float* dl = rowv[bsel][1];
      f32x16_t sc, dp;
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        sc[e] = 0.f;
        dp[e] = 0.f;
      }
      const int row = 32 * rb + l32;
  #pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        const int ch = (2 * s + g);
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(qt + row * C::ROWB + 16 * (ch ^ C::fb(row)));
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + krow * C::ROWB + 16 * (ch ^ C::fb(krow)));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf, sc, 0, 0, 0);
        const bf16x8_t da = *reinterpret_cast<const bf16x8_t*>(dt + row * C::ROWB + 16 * (ch ^ C::fb(row)));
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(vt + krow * C::ROWB + 16 * (ch ^ C::fb(krow)));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf, dp, 0, 0, 0);
      }
      bf16x8_t pb[2], db_[2];
  #pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int s0 = 32 * rb + 8 * q4 + 4 * g;
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
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
  #pragma unroll
        for (int dbk = 0; dbk < NDO; ++dbk) {
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
    };
    auto compute = [&](int n, int bsel, auto maskc) __attribute__((always_inline)) {
      const int tl = tile_of(n);
      const int t0 = bi.r0 + tl * TT;
      const int nv = (bi.r1 - t0 < TT ? bi.r1 - t0 : TT) * G;
      math(bsel, t0, nv, maskc);
    };

    // the key rows and the first tile, then one tile ahead: a tile's copies
    // are the only vector-memory operations in flight when it is awaited
    if (ntile > 0) issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    int n = 0;
    for (; n < nmask; ++n) {
      if (n + 1 < ntile) issue(n + 1, (n + 1) & 1);
      compute(n, n & 1, std::true_type{});
      wait_vmcnt<0>();
      __syncthreads();
    }
    for (; n < ntile; ++n) {
      if (n + 1 < ntile) issue(n + 1, (n + 1) & 1);
      compute(n, n & 1, std::false_type{});
      wait_vmcnt<0>();
      __syncthreads();
    }

    // The pair's partial sums, dV then dK: every wave stages its [32 keys][D]
    // block (16-byte chunk c of key row kr at c ^ (kr mod the row's chunks);
    // the loop's last barrier has retired every read of the LDS), then wave w
    // of the pair adds keys 16 (w / 4) .. +15 of both blocks into the fp32
    // accumulators, with consecutive lanes on consecutive floats, in a fixed
    // count of adds (a key past the item adds 0 to its last key).
    constexpr int SROW = D * 4;
    constexpr int SMASK = SROW / 16 - 1;
    static_assert(kWaves2 * 32 * SROW <= 2 * KVB + 4 * TILE, "staging fits");
    char* const stg = lds_all;  // wave w's block at w * 32 SROW
  #pragma unroll
    for (int which = 0; which < 2; ++which) {
      char* st = stg + wave * (32 * SROW);
  #pragma unroll
      for (int dbk = 0; dbk < NDO; ++dbk)
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t x = which == 0 ? f32x4_t{dv[dbk][4 * q4], dv[dbk][4 * q4 + 1], dv[dbk][4 * q4 + 2], dv[dbk][4 * q4 + 3]}
                                       : f32x4_t{dk[dbk][4 * q4], dk[dbk][4 * q4 + 1], dk[dbk][4 * q4 + 2], dk[dbk][4 * q4 + 3]};
          *reinterpret_cast<f32x4_t*>(st + l32 * SROW + 16 * ((8 * dbk + 2 * q4 + g) ^ (l32 & SMASK))) = x;
        }
      __syncthreads();
      const char* sa = stg + kw * (32 * SROW);        // rows 32 rb' + ..: the pair's rb = 0 wave
      const char* sb = stg + (kw + 4) * (32 * SROW);  // and its rb = 1 partner
      float* acc = which == 0 ? a.acc_v : a.acc_k;
      const int kbase = bi.k0 + 32 * kw + 16 * rb;
      constexpr int NI = 16 * D / 64;
      static_assert(NI % 8 == 0, "batches of 8");
  #pragma unroll 1
      for (int i0 = 0; i0 < NI; i0 += 8) {
        float x[8];
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int p = lane + 64 * (i0 + j);
          const int kr = 16 * rb + p / D;
          const int f = p % D;
          const int o = kr * SROW + 16 * ((f >> 2) ^ (kr & SMASK)) + 4 * (f & 3);
          x[j] = *reinterpret_cast<const float*>(sa + o) + *reinterpret_cast<const float*>(sb + o);
        }
  #pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int p = lane + 64 * (i0 + j);
          const int kk = kbase + p / D;
          const int f = p % D;
          const bool ok = kk < bi.k1;
          const int kc = ok ? kk : bi.k1 - 1;
          unsafeAtomicAdd(acc + ((size_t)kc * a.hkv + h_kv) * D + f, ok ? x[j] : 0.f);
        }
      }
      // the next staging (and a walking launch's next item) overwrite these areas
      __syncthreads();
    }
    if constexpr (!WALK) return;
  }  // items
}

// ------------------------------------------------------------- post pass
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

// workgroups per kv head of the dK/dV launch that walks the items past the
// host bound
constexpr int kBwdWalkPerHead = 4;

template <int D>
int launch_bwd_t(const BwdArgs& a, int64_t dq_blocks, int64_t dkdv_blocks, hipStream_t s) {
  int err = 0;
  // the dQ launch also forms the row terms, zeroes the dK / dV accumulators
  // and writes the item table (every flat layout with tokens has items)
  if (dq_blocks > 0) {
    if (a.seg_parent)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)dq_blocks), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)dq_blocks), dim3(kThreads), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
  }
  if constexpr (D <= 128) {
    if (dkdv_blocks > 0) {
      // the items the host bound predicts, one per workgroup, then any past it
      // (none when the bound holds: the walking workgroups then return at once)
      hipLaunchKernelGGL((bwd_dkdv2_kernel<D, false>), dim3((unsigned)dkdv_blocks), dim3(kThreads2), 0, s, a, 0);
      if ((err = (int)hipGetLastError())) return err;
      hipLaunchKernelGGL((bwd_dkdv2_kernel<D, true>), dim3((unsigned)(kBwdWalkPerHead * a.hkv)), dim3(kThreads2), 0,
                         s, a, (int)(dkdv_blocks / a.hkv));
      if ((err = (int)hipGetLastError())) return err;
    }
  }
  if constexpr (D >= 256) {
  constexpr int DO = 128;  // dK / dV columns per key-major launch
  for (int dofs = 0; dkdv_blocks > 0 && dofs < D; dofs += DO) {
    // the items the host bound predicts, one per workgroup ...
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DO, false>), dim3((unsigned)dkdv_blocks), dim3(kThreads), 0, s, a, 0,
                       dofs);
    if ((err = (int)hipGetLastError())) return err;
    // ... and any past it (none when the bound holds: the workgroups then find
    // their first item past the end and return)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DO, true>), dim3((unsigned)(kBwdWalkPerHead * a.hkv)), dim3(kThreads), 0,
                       s, a, (int)(dkdv_blocks / a.hkv), dofs);
    if ((err = (int)hipGetLastError())) return err;
  }
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
  if (d == 64) return launch_bwd_t<64>(a, dq_blocks, dkdv_blocks, s);
  if (d == 256) return launch_bwd_t<256>(a, dq_blocks, dkdv_blocks, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace psattn
