// psattn_flat.hip -- flat-packed prefix-shared attention forward (bf16), gfx950.
//
// PrefixSharing PR #50 ("设计简介", design summary) stores the shared prompt
// once, [P | S1 | ... | SN], and lets rollout token t of segment i see the
// prefix keys [0, P) and its own segment's keys up to t.  The planner turns
// that visibility into work items (a tile of query tokens inside the prefix
// or inside one rollout, stacked with the G query heads of one kv head); this
// kernel runs one item per workgroup:
//
//  * 4 waves x 32 stacked query rows; Q^T fragments stay in registers;
//  * the item's key ranges (the prefix, then the rollout's own keys) are
//    walked in 64-key tiles (the prefix's fully visible tiles last to first
//    in every other generation of a head's items, so that a generation
//    starts on the tiles its predecessor left in L2).  Each tile's K and V
//    rows are copied global -> LDS by global_load_lds_dwordx4 (no register
//    staging, no VALU), one tile ahead of the arithmetic in a double buffer;
//    the 16-byte chunks of a row land XOR-swizzled (the global address is
//    permuted, the LDS side is contiguous), so the operand reads below avoid
//    bank conflicts;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 K rows from LDS), so a
//    lane holds 16 scores of its own query row; online softmax in the log2
//    domain.  The reference maximum is moved lazily (see kTauFlat), and the
//    rescale of the accumulators is skipped when no row of the wave moved;
//  * O^T += V^T P^T with P^T taken from the score registers and V^T read from
//    the row-major V tile by ds_read_b64_tr_b16 (no transposed LDS writes).
//    The contraction order follows the score layout: position 8 g + e of the
//    16-key step ks is key 16 ks + 8 (e / 4) + 4 g + e % 4.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

#include <type_traits>

namespace psattn {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

#define PF_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))


// Lazy rescale: a row moves its reference maximum only when a tile's
// maximum exceeds it by more than kTauFlat (log2 units), so the weights stay
// <= 2^kTauFlat and the rescale of O (wave-wide, skipped unless some row
// moved) is rare after the first tiles.
constexpr float kTauFlat = 8.0f;
// Largest sum of one lane's 32 weights of a tile accepted without forming the
// tile's row maximum (so every weight is <= 2^16 relative to the reference).
constexpr float kSumCap = 65536.0f;

template <int D>
struct F2Cfg {
  static constexpr int BN = 64;                                   // keys per tile
  static constexpr int ROWB = 2 * D;                              // bytes of a K (or V) row
  static constexpr int CPR = ROWB / 16;                           // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;                          // K (or V) tile bytes
  static constexpr int NCOPY = TILE / 1024;                       // wave-wide 1 KiB copies per K (or V) tile
  static constexpr int CPW = 2 * NCOPY / kWaves;                  // copies per wave per tile (K + V)
  static constexpr int NSTEP = D / 16;                            // k-steps of the score product
  static constexpr int NDB = D / 32;                              // 32-column output blocks
  static constexpr int MINB = D >= 256 ? 1 : 2;
  static_assert(2 * NCOPY % kWaves == 0, "copies split evenly over the waves");
  __device__ static constexpr int fk(int r) { return r & (CPR - 1); }
  // V rows: a 32-lane pass of the transposed reads covers 4 rows x 4 chunks;
  // the swizzle spreads them over all 64 banks (rows of 128 bytes already
  // alternate bank halves, so there only row pairs are separated)
  __device__ static constexpr int fv(int r) { return CPR >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// CHAIN: multi-level sharing (PrefixSharing PR #50, mask construction, the
// multi-level tree "chain" case: a rollout continues a parent segment, which
// may continue another).  After the prefix and the item's own range, one more
// pass per ancestor segment walks that segment's keys, all visible, carrying
// the online-softmax state.  A compile-time variant, so that one-level
// sharing keeps its own code.
template <int D, bool CHAIN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(F2Cfg<D>::MINB)))
void flat2_kernel(FlatArgs a) {
  using C = F2Cfg<D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][C::TILE];  // [buffer][K, V]

  const int blk = blockIdx.x;
  const int h_kv = blk % a.hkv;
  const int j = blk / a.hkv;
  const Item it = flat_item(j, h_kv, a.prefix_len, a.nseg, a.seg_offsets, a.tile_tokens);
  if (it.kind == kNone) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // stacked row of this lane's query column: token-major, heads interleaved
  const int r = wave * kWaveRows + l32;
  const int tok = r / a.g;
  const int hl = r - tok * a.g;
  const int token = it.q_begin + tok;
  const bool valid = (tok < a.tile_tokens) && (token < it.q_end);
  const int token_c = valid ? token : it.q_begin;
  const size_t qrow = (size_t)token_c * a.hq + h_kv * a.g + hl;

  // Q^T fragments: k-step s, lane group g holds d = 16 s + 8 g .. +8
  bf16x8_t qf[C::NSTEP];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + qrow * D;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) qf[s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(qp + 16 * s + 8 * g));
  }

  // Tiles of a range that are whole and end at or before the item's first
  // query token are visible to every row: they form a leading run of the
  // range.  They are walked first (no mask), then the rest of both ranges.
  // (With CHAIN, later passes put an ancestor segment's range in r0 and
  // leave r1 empty.)
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
  // The workgroup slots of one kv head (two per CU, spread over the CUs its
  // XCDs hold) take its items in order, one generation of items at a time;
  // odd generations walk the clean tiles of the first range (the prefix)
  // last to first, so that each generation starts on the tiles the one
  // before it read last, still in L2.  The order of the keys does not change
  // the result (online softmax).
  const int head_slots = (256 * C::MINB) / a.hkv > 0 ? (256 * C::MINB) / a.hkv : 1;
  const bool rev = ((j / head_slots) & 1) != 0;
  auto tile_range = [&](int n, int& k0, int& ke) __attribute__((always_inline)) {
    if (n < c0) {
      k0 = r0b + (rev ? c0 - 1 - n : n) * BN;
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

  // This wave's copies of a tile: copy q = wave * CPW + t is 1 KiB block jb of
  // the K tile (q < NCOPY) or of the V tile.  Lane l of a block carries chunk
  // pos of tile row `row` (p = 64 jb + l); its byte offset inside the tile's
  // rows is fixed, so it is computed once.
  const bool w_isv = wave * C::CPW >= C::NCOPY;  // a wave's copies are all K or all V
  const char* wbase = w_isv ? vbase : kbase;
  uint32_t coff[C::CPW];
#pragma unroll
  for (int t = 0; t < C::CPW; ++t) {
    const int jb = (wave * C::CPW + t) % C::NCOPY;
    const int p = jb * 64 + lane;
    const int row = p / C::CPR;
    const int pos = p % C::CPR;
    coff[t] = (uint32_t)row * row_stride + 16u * (uint32_t)(pos ^ (w_isv ? C::fv(row) : C::fk(row)));
  }
  // copies of tile n into LDS buffer B; rows past the range end repeat its
  // last row (finite data, masked in the arithmetic)
  auto issue = [&](int n, int bsel) __attribute__((always_inline)) {
    const uint32_t bofs = (uint32_t)bsel * (2 * C::TILE);
    int k0, ke;
    tile_range(n, k0, ke);
    const char* base = wbase + (size_t)k0 * row_stride;
    if (k0 + BN <= ke) {
#pragma unroll
      for (int t = 0; t < C::CPW; ++t) {
        const int jb = (wave * C::CPW + t) % C::NCOPY;
        dma16_s(base, coff[t], lds_addr(&smem[0][w_isv ? 1 : 0][jb * 1024]) + bofs);
      }
    } else {
      const int lastr = ke - 1 - k0;
#pragma unroll
      for (int t = 0; t < C::CPW; ++t) {
        const int jb = (wave * C::CPW + t) % C::NCOPY;
        const int p = jb * 64 + lane;
        const int row = p / C::CPR;
        const int pos = p % C::CPR;
        const int rc = row < lastr ? row : lastr;
        const uint32_t off = (uint32_t)rc * row_stride + 16u * (uint32_t)(pos ^ (w_isv ? C::fv(row) : C::fk(row)));
        dma16_s(base, off, lds_addr(&smem[0][w_isv ? 1 : 0][jb * 1024]) + bofs);
      }
    }
  };

  float m_run = kNegBig;
  float l_run = 0.f;
  f32x16_t o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  const float c = a.scale_log2;

  // MASK: the tile crosses the range end or the causal diagonal
  auto math = [&](const char* kt, const char* vt, int key0, int kend, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    // ---- S^T for keys 32 kb + (0..31): lane (l32, g), reg i holds key
    // 32 kb + 8 (i / 4) + 4 g + i % 4 of query row l32
    f32x16_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      const int row = 32 * kb + l32;
      const char* krow = kt + row * C::ROWB;
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((2 * s + g) ^ C::fk(row)));
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sc[kb], 0, 0, 0);
      }
    }
    float mr = -__builtin_inff();
    if constexpr (MASK) {
      // visible keys of this row: key < kend and key <= token
      const int lim = (kend < token + 1 ? kend : token + 1) - key0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          sc[kb][i] = kr < lim ? sc[kb][i] : -__builtin_inff();
        }
    }
    // Weights against the current reference maximum, without forming the
    // tile's row maximum first.  The lane's sum of its 32 weights bounds each
    // of them; while it stays at or below kSumCap no weight can overflow and
    // the tile is done.  Otherwise (the first tile of a row, whose reference
    // is still kNegBig, or a score far above the reference) the row maximum
    // is formed, the reference moved lazily as before, and the weights taken
    // again.  (The sum is of the fp32 weights: summing their bf16 roundings
    // instead moves the LSE by up to 2^-9 when one key dominates.)
    bf16x8_t pt[4];  // k-step ks = 2 kb + half: regs 8 half .. 8 half + 7 of sc[kb]
    float psum;
    auto weights = [&]() __attribute__((always_inline)) {
      psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(sc[kb][i], c, -m_run));
          pt[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
          psum += p;
        }
    };
    weights();
    if (__builtin_amdgcn_ballot_w64(!(psum <= kSumCap)) != 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mr = fmaxf(mr, sc[kb][i]);
      mr = max_xor32(mr);
      const float mx = mr * c;
      const bool grow = mx > m_run + kTauFlat;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float mn = grow ? mx : m_run;
        const float al = fast_exp2(m_run - mn);
        l_run *= al;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) o[db] *= al;
        m_run = mn;
      }
      weights();
    }
    l_run += psum;
    // ---- O^T += V^T P^T: A operand lane (d, g) = V rows 16 ks + 8 t + 4 g + 0..3
    // of column d (t = 0, 1), by ds_read_b64_tr_b16: in-group source lane
    // ap + 4 sp addresses row 16 ks + 8 t + 4 g + sp, columns 4 ap .. +3
    const int li = lane & 15;
    const int sp = li >> 2;
    const int ap = li & 3;
    const int hgrp = l32 >> 4;
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
              PF_LDS_PTR(s16x4_t, vt + row * C::ROWB + 16 * (chunk ^ C::fv(row)) + 8 * (ap & 1)));
        }
        const s16x8_t v8 = {vv[0][0], vv[0][1], vv[0][2], vv[0][3], vv[1][0], vv[1][1], vv[1][2], vv[1][3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, v8), pt[ks], o[db], 0, 0, 0);
      }
    }
  };

  auto compute = [&](int n, auto maskc) __attribute__((always_inline)) {
    int k0, ke;
    tile_range(n, k0, ke);
    math(smem[n & 1][0], smem[n & 1][1], k0, ke, maskc);
  };

  // retire the query loads before the copies start: the copies are waited for
  // with explicit vmcnt counts that the compiler does not know about
#pragma unroll
  for (int s = 0; s < C::NSTEP; ++s) asm volatile("" ::"v"(qf[s]));
  int anc = CHAIN && it.kind == kFlatSuffix && a.seg_parent ? a.seg_parent[it.seg] : -1;
  int child = it.seg;
  for (;;) {
    if (nt > 0) issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    int n = 0;
    // the clean run two tiles per pass, so that each tile's LDS buffer is a
    // compile-time constant (its operand addresses fold into the reads'
    // immediate offsets: 18 fewer VALU instructions per tile); at D = 256 the
    // second copy of the tile body costs spills, so there one per pass
    for (; D <= 128 && n + 1 < nc; n += 2) {
      issue(n + 1, 1);
      {
        int k0, ke;
        tile_range(n, k0, ke);
        math(smem[0][0], smem[0][1], k0, ke, std::false_type{});
      }
      wait_vmcnt<0>();
      __syncthreads();
      if (n + 2 < nt) issue(n + 2, 0);
      {
        int k0, ke;
        tile_range(n + 1, k0, ke);
        math(smem[1][0], smem[1][1], k0, ke, std::false_type{});
      }
      wait_vmcnt<0>();
      __syncthreads();
    }
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
    }
  }

  // ---- epilogue.  O = acc / l goes through LDS so that every global store
  // is a whole 16-byte chunk of a row: the rows leave as full cache lines,
  // written non-temporally (they are not read again here, and kept in L2 they
  // would evict the prefix K/V the other items of this head still read).
  // Each wave stages its 32 rows (chunk c of row r at c ^ (r % CPR)) in the
  // tiles, which every wave is done with after the loop's last barrier.
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  char* ost = &smem[0][0][0] + wave * (kWaveRows * C::ROWB);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // columns 32 db + 8 g4 + 4 g .. +3: half g of chunk 4 db + g4
      const u32x2_t v = {pack_bf16x2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                         pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
      *reinterpret_cast<u32x2_t*>(ost + l32 * C::ROWB + 16 * ((4 * db + g4) ^ (l32 & (C::CPR - 1))) + 8 * g) = v;
    }
  }
  if (valid && g == 0) a.lse[qrow] = (m_run + fast_log2(lt)) * kLn2;
  __syncthreads();
  constexpr int NOUT = kWaveRows * C::CPR / 64;  // 16-byte stores per lane
  // every staged chunk is read first (in bounds whatever the row), so that the
  // reads issue together instead of one round trip behind each row's test
  u32x4_t x[NOUT];
#pragma unroll
  for (int k = 0; k < NOUT; ++k) {
    const int p = 64 * k + lane;
    const int row = p / C::CPR;
    const int ch = p % C::CPR;
    x[k] = *reinterpret_cast<const u32x4_t*>(ost + row * C::ROWB + 16 * (ch ^ (row & (C::CPR - 1))));
  }
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
      __bf16* op = reinterpret_cast<__bf16*>(a.o) + ((size_t)tkn * a.hq + h_kv * a.g + hh) * D + 8 * ch;
      __builtin_nontemporal_store(x[k], reinterpret_cast<u32x4_t*>(op));
    }
  }
}

template <int D>
int launch_t(const FlatArgs& a, int64_t n_blocks, hipStream_t s) {
  if (a.seg_parent)
    hipLaunchKernelGGL((flat2_kernel<D, true>), dim3((unsigned)n_blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((flat2_kernel<D, false>), dim3((unsigned)n_blocks), dim3(kThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_flat_bf16(const FlatArgs& a, int d, int64_t n_blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (d) {
    case 64: return launch_t<64>(a, n_blocks, s);
    case 128: return launch_t<128>(a, n_blocks, s);
    case 256: return launch_t<256>(a, n_blocks, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace psattn
