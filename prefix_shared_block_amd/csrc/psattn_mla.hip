// psattn_mla.hip -- sparse shared-latent MLA forward (bf16), gfx950.
//
// DSA / sparse-MLA prefill (the vLLM issue "[Perf] SM8x sparse-MLA prefill
// fallback re-reads the shared MLA latent once per head", sections 适用环境
// and 原因分析): every query token attends to the cached tokens its top-k list
// names, and all of its heads read the same 512-wide latent rows, which are
// the keys and the values alike (no rope part).  The page's kernel ran one
// program per (token, head), re-reading the latent rows for every head, and
// its measurements credit 2-D (heads x dims) tiles for the speed-up.  Here a
// workgroup takes one token with all H of its heads:
//
//  * the token's list is staged in LDS and compacted in order (entries
//    outside [0, num_kv) dropped, one wave ballot per round), so that every
//    16-key tile but the last is full and needs no mask;
//  * each tile's 16 latent rows are gathered global -> LDS with
//    global_load_lds_dwordx4, one 1 KiB row per wave instruction, three
//    tiles ahead in a ring of four buffers.  Row r's chunks land XOR-swizzled
//    by r & 15; the tile is read both ways (it is K and V at once), as rows
//    by the score product and transposed by the value product, and the key
//    order of the value product (key_of) keeps the transposed reads free of
//    bank conflicts too;
//  * H / 16 waves.  Scores: wave w takes heads 16 w .. 16 w + 15 (their Q^T
//    fragments stay in registers), S^T = C Q^T on v_mfma_f32_16x16x32_bf16,
//    online softmax in the log2 domain with a lazily moved reference maximum;
//    it leaves P (bf16) and the heads' rescale factors in LDS.  Values: wave w
//    takes 512 / (H / 16) latent dims of every head, O^T += C^T P^T on
//    v_mfma_f32_32x32x16_bf16, reading only its dims of the tile.  So the
//    accumulators are split by dims and the query fragments by heads: each
//    wave holds 128 accumulator and 64 fragment registers whatever H is;
//  * the optional per-head sink logit joins the normaliser in the epilogue;
//  * dense causal variant (no list): the query tokens are the cache's last
//    rows and token t takes rows 0 .. S - T + t, in order, with the same
//    tiles, gathers and products.
#include "device_common.h"
#include "mla.h"

#include <type_traits>

namespace psattn {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

#define PM_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kBN = 16;                    // keys per tile
constexpr int kNBuf = 4;                   // tile buffers: tiles are gathered kNBuf - 1 ahead
static_assert(kNBuf >= 2 && kNBuf <= 4, "waits cover up to two tiles in flight");
constexpr int kRowB = 2 * kMlaDim;         // bytes of a latent row (1 KiB)
constexpr int kTile = kBN * kRowB;         // 16 KiB
constexpr int kNStep = kMlaDim / 32;       // k-steps of the score product (16x16x32)
constexpr int kPRow = 2 * kBN + 8;         // bytes per head row of P in LDS (padded)
constexpr float kTau = 8.0f;               // lazy rescale threshold (log2 units)
constexpr float kLog2e = 1.4426950408889634f;

// Chunk swizzle of tile row r: chunk c of the row sits at c ^ (r & 15).
__device__ __forceinline__ int fsw(int r) { return r & 15; }

// Key order of the value product inside a 16-key block.  Position
// i = 8 g + 4 u + e of its contraction (and of P in LDS) is key
// 4 e + 2 u + g: the four rows that one transposed read gathers (e = 0..3)
// then differ in bits 2..3, which keeps those reads free of bank conflicts
// under the swizzle above.  (The score product reads its rows in key order,
// lane i row i, the one order measured free of conflicts for its 16-byte row
// reads; its results are scattered to their positions when P is stored.)
__device__ __forceinline__ int key_of(int i) { return 4 * (i & 3) + 2 * ((i >> 2) & 1) + (i >> 3); }
__device__ __forceinline__ int pos_of(int k) { return (k >> 2) + 4 * ((k >> 1) & 1) + 8 * (k & 1); }

// NW = H / 16 waves.  Wave w: score heads 16 w .. +15; value dims
// DW w .. DW (w + 1) with DW = 512 / NW, for head blocks 0 .. HB - 1.
// DENSE: no list; the tokens are the cache's last rows and token t takes
// rows 0 .. num_kv - num_tokens + t in order (a causal prefill).
template <int NW, bool DENSE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void mla_sparse_kernel(MlaArgs a) {
  constexpr int H = 16 * NW;
  constexpr int NT = 64 * NW;
  constexpr int HB = H / 32;               // 32-head blocks of the value product
  constexpr int NDBW = kMlaDim / 32 / NW;  // 32-dim blocks per wave
  constexpr int PER = kMlaMaxTopk / NT;    // list entries per thread
  constexpr int RPW = kBN / NW;            // tile rows gathered per wave
  static_assert(HB * NDBW == 8, "eight accumulator blocks per wave");
  __shared__ __attribute__((aligned(1024))) char smem[kNBuf][kTile];
  __shared__ __attribute__((aligned(16))) int sidx[kMlaMaxTopk];
  // P [head][position] bf16, the heads' rescale factors (1 / l at the end) and
  // the waves' "some head moved" flags, double-buffered by tile parity
  __shared__ __attribute__((aligned(16))) char sp_[2][H * kPRow];
  __shared__ float salpha[2][H];
  __shared__ int smoved[2][NW];
  __shared__ int wcnt[NW];

  // later tokens list more keys (a causal prefill): they start first
  const int t = a.num_tokens - 1 - (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int shead = wave * 16 + l16;       // this lane's score head

  // Q^T fragments: k-step s, lane group g4 holds dims 32 s + 8 g4 .. +8
  bf16x8_t qf[kNStep];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + ((size_t)t * H + shead) * kMlaDim;
#pragma unroll
    for (int s = 0; s < kNStep; ++s)
      qf[s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(qp + 32 * s + 8 * g4));
  }
  int cnt = 0;
  if constexpr (DENSE) {
    cnt = a.num_kv - a.num_tokens + t + 1;
  } else {
    // the list: thread tid holds entries tid + NT r
    int ent[PER];
    {
      const int32_t* ip = a.indices + (size_t)t * a.topk;
      const int elast = a.topk > 0 ? a.topk - 1 : 0;
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int e = tid + NT * r;
        const int v = a.topk > 0 ? ip[e < elast ? e : elast] : -1;
        ent[r] = e < a.topk ? v : -1;
      }
    }
    // compaction, in list order: round r places the valid entries of
    // tid + NT r after those of the earlier rounds and lower threads
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const bool ok = (unsigned)ent[r] < (unsigned)a.num_kv;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (lane == 0) wcnt[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int before = cnt, total = cnt;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cw = wcnt[w];
        before += w < wave ? cw : 0;
        total += cw;
      }
      if (ok) sidx[before + below] = ent[r];
      cnt = __builtin_amdgcn_readfirstlane(total);
      __syncthreads();
    }
  }
  const int ntile = (cnt + kBN - 1) / kBN;
  const int nfull = cnt / kBN;
  const int last_id = DENSE ? cnt - 1 : (cnt > 0 ? __builtin_amdgcn_readfirstlane(sidx[cnt - 1]) : 0);

  const char* cbase = reinterpret_cast<const char*>(a.ckv);
  const size_t rstride = (size_t)a.kv_stride * 2;
  // this wave's rows of tile n into buffer b; positions past the list's end
  // repeat its last row (finite data, masked in the arithmetic)
  auto issue = [&](int n, int b) __attribute__((always_inline)) {
    const uint32_t lbase = lds_addr(&smem[b][0]);
    const int k0 = n * kBN + wave * RPW;
    int ids[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) ids[i] = DENSE ? k0 + i : sidx[k0 + i];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = wave * RPW + i;
      const int idr = __builtin_amdgcn_readfirstlane(ids[i]);
      const int id = k0 + i < cnt ? idr : last_id;
      dma16_s(cbase + (size_t)id * rstride, 16u * (uint32_t)(lane ^ fsw(r)), lbase + (uint32_t)r * kRowB);
    }
  };

  float m_run = kNegBig;  // score head shead (the same in its four lanes)
  float l_run = 0.f;      // this lane's part of the head's sum
  f32x16_t o[NDBW][HB];   // O^T blocks: dims 32 (NDBW wave + db) .., heads 32 hb ..
#pragma unroll
  for (int db = 0; db < NDBW; ++db)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][hb][e] = 0.f;
  const float c = a.scale_log2;

  // ---- scores of tile kt for this wave's heads -> P and rescale factors in
  // LDS.  Lane (l16, g4), register e of block kb holds key 16 kb + 4 g4 + e;
  // P is stored by position (pos_of).
  auto scores = [&](const char* kt, int nvalid, int pb, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    f32x4_t sc[kBN / 16];
#pragma unroll
    for (int kb = 0; kb < kBN / 16; ++kb) {
      sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * kb + l16;
      const char* krow = kt + row * kRowB;
      const int sw = fsw(row);
#pragma unroll
      for (int s = 0; s < kNStep; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((4 * s + g4) ^ sw));
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc[kb], 0, 0, 0);
      }
    }
    float mr = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < kBN / 16; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (MASK) {
          if (16 * kb + 4 * g4 + e >= nvalid) sc[kb][e] = -__builtin_inff();
        }
        mr = fmaxf(mr, sc[kb][e]);
      }
    mr = max_xor32(max_xor16(mr));  // the head's four lane groups
    const float mx = mr * c;
    const bool grow = mx > m_run + kTau;
    float al = 1.f;
    if (grow) {
      al = fast_exp2(m_run - mx);
      l_run *= al;
      m_run = mx;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBN / 16; ++kb) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(sc[kb][e], c, -m_run));
        psum += p[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<__bf16*>(&sp_[pb][shead * kPRow + 2 * (16 * kb + pos_of(4 * g4 + e))]) = (__bf16)p[e];
    }
    l_run += psum;
    if (g4 == 0) salpha[pb][shead] = al;
    if (lane == 0) smoved[pb][wave] = __builtin_amdgcn_ballot_w64(grow) != 0;
  };

  // ---- O^T += C^T P^T for this wave's dims.  Position 8 g + 4 u + e of
  // 16-key step ks is key 16 ks + key_of(8 g + 4 u + e), for the A operand
  // (rows of the tile, read transposed: source lane ap + 4 e of a 16-lane
  // group addresses that row) and the B operand (P, stored by position).
  auto values = [&](const char* kt, int par) __attribute__((always_inline)) {
    int moved = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) moved |= smoved[par][w];
    if (moved) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float al = salpha[par][32 * hb + l32];
#pragma unroll
        for (int db = 0; db < NDBW; ++db) o[db][hb] *= al;
      }
    }
    const int li = lane & 15;
    const int sp = li >> 2;
    const int ap = li & 3;
    const int hgrp = l32 >> 4;
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks) {
      bf16x8_t pb[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const char* prow = &sp_[par][(32 * hb + l32) * kPRow + 2 * (16 * ks + 8 * g)];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(prow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(prow + 8);
        const u32x4_t both = {lo[0], lo[1], hi[0], hi[1]};
        pb[hb] = __builtin_bit_cast(bf16x8_t, both);
      }
#pragma unroll
      for (int db = 0; db < NDBW; ++db) {
        s16x4_t vv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 16 * ks + key_of(8 * g + 4 * u + sp);
          const int chunk = 4 * (NDBW * wave + db) + 2 * hgrp + (ap >> 1);
          vv[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              PM_LDS_PTR(s16x4_t, kt + row * kRowB + 16 * (chunk ^ fsw(row)) + 8 * (ap & 1)));
        }
        const s16x8_t v8 = {vv[0][0], vv[0][1], vv[0][2], vv[0][3], vv[1][0], vv[1][1], vv[1][2], vv[1][3]};
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, v8);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          o[db][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[hb], o[db][hb], 0, 0, 0);
      }
    }
  };

  // retire the query loads before the copies start: the copies are waited for
  // with explicit vmcnt counts that the compiler does not know about
#pragma unroll
  for (int s = 0; s < kNStep; ++s) asm volatile("" ::"v"(qf[s]));
  // wait until tile m has landed, when the tiles up to `last` are issued
  // (copies complete in issue order, RPW per tile and wave)
  auto wait_tile = [&](int m, int last) __attribute__((always_inline)) {
    const int later = last - m;
    if (later <= 0) wait_vmcnt<0>();
    else if (kNBuf > 2 && later == 1) wait_vmcnt<RPW>();
    else wait_vmcnt<2 * RPW>();
  };
  // One barrier per tile: iteration n runs the values of tile n (its P was
  // left by the previous iteration) and then the scores of tile n + 1, whose
  // rows every wave awaited before that barrier; P, the rescale factors and
  // the flags alternate between two buffers.
  auto score_tile = [&](int m) __attribute__((always_inline)) {
    const char* kt = smem[m % kNBuf];
    if (m < nfull)
      scores(kt, kBN, m & 1, std::false_type{});
    else
      scores(kt, cnt - m * kBN, m & 1, std::true_type{});
  };
  const int lastp = (ntile < kNBuf - 1 ? ntile : kNBuf - 1) - 1;  // tiles issued up front
#pragma unroll
  for (int p = 0; p < kNBuf - 1; ++p)
    if (p < ntile) issue(p, p);
  wait_tile(0, lastp);
  __syncthreads();
  if (ntile > 0) score_tile(0);
  wait_tile(1, lastp);
  __syncthreads();
  for (int n = 0; n < ntile; ++n) {
    const int nx = n + kNBuf - 1;
    if (nx < ntile) issue(nx, nx % kNBuf);
    values(smem[n % kNBuf], n & 1);
    if (n + 1 < ntile) score_tile(n + 1);
    wait_tile(n + 2, nx < ntile - 1 ? nx : ntile - 1);
    __syncthreads();
  }

  // ---- epilogue: the sink joins the normaliser; the score waves leave
  // 1 / l per head in LDS for the value waves
  {
    const float lt = l_run + __shfl_xor(l_run, 16) + __shfl_xor(l_run, 32) + __shfl_xor(l_run, 48);
    float mf = m_run, so = 1.f, den = lt;
    if (a.sink) {
      const float s2 = a.sink[shead] * kLog2e;
      mf = fmaxf(m_run, s2);
      so = fast_exp2(m_run - mf);
      den = __builtin_fmaf(lt, so, fast_exp2(s2 - mf));
    }
    if (g4 == 0) {
      salpha[0][shead] = den > 0.f ? so / den : 0.f;
      a.lse[(size_t)t * H + shead] = den > 0.f ? (mf + fast_log2(den)) * kLn2 : -__builtin_inff();
    }
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 32 * hb + l32;
    const float inv = salpha[0][head];
    __bf16* op = reinterpret_cast<__bf16*>(a.o) + ((size_t)t * H + head) * kMlaDim;
#pragma unroll
    for (int db = 0; db < NDBW; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // dims 32 (NDBW wave + db) + 8 q4 + 4 g .. +3
        const int d0 = 32 * (NDBW * wave + db) + 8 * q4 + 4 * g;
        const u32x2_t v = {pack_bf16x2(o[db][hb][4 * q4] * inv, o[db][hb][4 * q4 + 1] * inv),
                           pack_bf16x2(o[db][hb][4 * q4 + 2] * inv, o[db][hb][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + d0) = v;
      }
    }
  }
}

template <int NW>
int launch_w(const MlaArgs& a, bool dense, hipStream_t s) {
  if (dense)
    hipLaunchKernelGGL((mla_sparse_kernel<NW, true>), dim3((unsigned)a.num_tokens), dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((mla_sparse_kernel<NW, false>), dim3((unsigned)a.num_tokens), dim3(64 * NW), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_mla(const MlaArgs& a, bool dense, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dense && (a.num_kv < a.num_tokens || a.indices)) return (int)hipErrorInvalidValue;
  switch (a.num_heads) {
    case 32: return launch_w<2>(a, dense, s);
    case 64: return launch_w<4>(a, dense, s);
    case 128: return launch_w<8>(a, dense, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace psattn
