// psattn_regstream.hip -- register-streamed split-KV verify pass for
// speculative verify with few stacked query rows (draft_len * G <= 16),
// bf16 or OCP fp8 e4m3fn K/V in a paged cache, gfx950.
//
// sglang PR #27382 ("实现拆解", implementation breakdown) splits the verify
// path into a first stage that walks the long paged prefix in splits and
// writes one partial (O, LSE) per split, and a second stage that merges the
// splits with the small causal draft block.  For the shapes where HBM
// bandwidth is the only real bound (16 rows against thousands of keys: 16
// flop per byte) this file does both, arranged for HBM streaming:
//
//  * paged_reg_kernel: one workgroup per (request, kv head, split), of
//    reg_waves(D) waves (8 up to D = 128, 4 at D = 256), each streaming its
//    own contiguous run of the split's stages with no barrier until the
//    waves' results are merged in LDS at the end.  The last split of each
//    (request, kv head) also runs the causal draft block as one extra 16-key
//    stage (draft row j sees draft keys 0..j), so its partial already
//    contains it;
//  * paged_merge_kernel: one wave per (stacked row, 64 columns) merges the
//    splits' partial results by log-sum-exp and applies v_scale.
//
//  * keys are walked in 16-key stages.  A stage is one aligned 16-slot block
//    of one page, so its page id and base address are wave-uniform (scalar
//    registers, the page id read with a scalar load) and every lane's byte
//    offset inside the page is fixed;
//  * loads go straight into registers (plain vector loads sustain more of the
//    HBM bandwidth than the direct global->LDS path on this part), into a
//    ring of NB register sets; a set is reloaded NB stages ahead as soon as
//    its rows have been written to LDS, before the stage's arithmetic.
//    Each wave-wide 16-byte load covers whole key rows (consecutive lanes
//    read consecutive 16-byte chunks of a row): reading every row in 64-byte
//    pieces spread over four loads measured markedly slower;
//  * the stage is then written (as bf16; fp8 codes converted exactly, once
//    per element) to a wave-private LDS tile pair and read back in MFMA
//    operand order: K rows with ds_read_b128 as the A operand of
//    v_mfma_f32_16x16x32_bf16 for S^T = K Q^T, V columns with the transpose
//    read ds_read_b64_tr_b16 as the A operand of v_mfma_f32_16x16x16_bf16 for
//    O^T += V^T P^T, whose B operand P^T is the score registers themselves.
//    The tiles are private to the wave, so the stage loop needs no barrier;
//  * k_scale is folded into the logit scale and v_scale is applied by the
//    combine stage;
//  * online softmax in the log2 domain with lazy rescaling (the running
//    maximum only moves when a row's new maximum exceeds it by more than
//    kTau, so every exp2 argument stays <= kTau);
//  * the split's normalised partial O is stored in bf16 (its LSE in fp32):
//    half the bytes written here and read back by the merge.
//
// LDS tiles are row-major [16 keys][D bf16] with 16-byte chunks XOR-swizzled
// per row (K: chunk ^ (row % CPR); V: chunk ^ (2 row % CPR)).
// Keys past the end of the prefix in the last stage are loaded from the last
// valid slot (finite data) and masked to -inf, so their probability is 0.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace psattn {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

#define PR_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

template <int D, int KDT>
struct RCfg {
  static constexpr int ES = Elem<KDT>::size;
  static constexpr int ROWB = D * ES;    // global bytes of one key row of one kv head
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per global row
  static constexpr int RPI = 64 / CPR;   // key rows covered by one wave-wide load
  static constexpr int NLD = 16 / RPI;   // loads per lane for a 16-key K (or V) tile
  static constexpr int TROWB = 2 * D;    // LDS row bytes (bf16)
  static constexpr int TCPR = TROWB / 16;
  static constexpr int TILE = 16 * TROWB;
  static constexpr int NSTEP = D / 32;   // k-steps of the score product
  static constexpr int NDB = D / 16;     // 16-column blocks of the output
  // register sets in the ring: about 128 VGPRs of K/V in flight per lane
  static constexpr int NB = (512 / (2 * NLD * 16)) >= 4 ? 4 : (512 / (2 * NLD * 16));
  static_assert(CPR <= 64 && NLD >= 1 && NB >= 2, "shape");
  __device__ static constexpr int fk(int r) { return r & (TCPR - 1); }
  __device__ static constexpr int fv(int r) { return (2 * r) & (TCPR - 1); }
};

// 16 bytes of a global row (chunk pos) -> the row's LDS tile slot(s), as bf16
template <int KDT, int TCPR>
__device__ __forceinline__ void put_chunk(char* trow, int pos, int f, const u32x4_t x) {
  if constexpr (KDT == DT_BF16) {
    *reinterpret_cast<u32x4_t*>(trow + 16 * (pos ^ f)) = x;
  } else {
    u32x4_t lo, hi;
    fp8x16_to_bf16(x, lo, hi);
    *reinterpret_cast<u32x4_t*>(trow + 16 * ((2 * pos) ^ f)) = lo;
    *reinterpret_cast<u32x4_t*>(trow + 16 * ((2 * pos + 1) ^ f)) = hi;
  }
}

// W waves per workgroup, each streaming its own share of the split's stages
// independently; OCC: waves per SIMD the register budget is held to (2 for
// head dims up to 128, so that two independent streams share each SIMD).
// TREE: the draft block follows the request's draft mask (a compile-time
// variant, so that the causal kernel keeps its own code)
template <int D, int KDT, int OCC, int W, bool TREE>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(OCC)))
void paged_reg_kernel(PagedArgs a) {
  using C = RCfg<D, KDT>;
  constexpr int NB = C::NB;
  constexpr int NLD = C::NLD;
  // per wave: [buffer][K, V] tiles; reused at the end for the wave's partial
  // result (16 rows x D floats, then 16 running maxima and 16 sums)
  static_assert(16 * D * 4 + 2 * 16 * 4 <= 4 * C::TILE, "merge area");
  __shared__ __attribute__((aligned(16))) char tiles_all[W][2][2][C::TILE];

  const Item it = paged_item(blockIdx.x, a.hkv, a.n_splits, a.split_len, a.draft_len, a.prefix_lens);
  const int b = it.seg;
  const int h_kv = it.h_kv;
  const int qb = draft_base(a.qo_indptr, b, a.draft_len);  // the request's first draft row
  const int qn = draft_count(a.qo_indptr, b, a.draft_len);  // and its number of draft rows
  if (qn <= 0) return;                                       // a request without draft rows
  const int wave = W == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  char (*tiles)[2][C::TILE] = tiles_all[wave];
  const int lane = threadIdx.x & 63;
  const int q16 = lane & 15;
  const int g = lane >> 4;
  const int pos = lane % C::CPR;  // load layout: chunk pos of key row RPI j + rr
  const int rr = lane / C::CPR;
  const int ps_shift = __builtin_ctz((unsigned)a.page_size);
  const int ps_mask = a.page_size - 1;
  // the page table is read through the constant address space: a uniform
  // load from it is always a scalar load (s_load), never a vector one
  typedef const __attribute__((address_space(4))) int32_t* ctab_t;
  const ctab_t ptab = reinterpret_cast<ctab_t>(reinterpret_cast<uintptr_t>(a.kv_indices + a.kv_indptr[b]));
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const uint32_t slot_stride = (uint32_t)a.hkv * C::ROWB;
  const size_t page_bytes = (size_t)slot_stride << ps_shift;
  const size_t head_off = (size_t)h_kv * C::ROWB;
  // The split's 16-key stages are dealt to the waves as contiguous runs (the
  // first runs one longer); the last wave of the last split also runs the
  // draft block as one more stage.
  const int sp_stages = (it.r0_end - it.r0_begin + 15) >> 4;
  const int per = sp_stages / W;
  const int rem = sp_stages - per * W;
  const int first = wave * per + (wave < rem ? wave : rem);
  const int npre = per + (wave < rem ? 1 : 0);
  const int kbeg = it.r0_begin + 16 * first;
  const int kend = npre > 0 ? (kbeg + 16 * npre < it.r0_end ? kbeg + 16 * npre : it.r0_end) : kbeg;
  const int nst = npre + (it.split == a.n_splits - 1 && wave == W - 1 ? 1 : 0);
  // draft block: row j of request b at k_ext + ((b L + j) Hkv + h_kv) * ROWB,
  // the same row stride as the slots of a page
  const size_t ext_off = ((size_t)qb * a.hkv + h_kv) * C::ROWB;
  const int trow = q16 / a.g;  // draft position of stacked row q16
  // draft keys 4 g + e (e = 0..3) this lane's row sees: its draft-mask row,
  // or the causal chain (keys 0 .. trow)
  uint32_t dvis = 0;
  if constexpr (TREE) {
    const int tr = trow < qn ? trow : qn - 1;
    const uint8_t* mrow = a.draft_mask + ((size_t)b * a.draft_len + tr) * a.draft_len;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * g + e;
      const bool v = j < qn && mrow[j] != 0;
      dvis |= (v ? 1u : 0u) << e;
    }
    asm volatile("" ::"v"(dvis));  // retired here, before the stage ring
  }

  // ---- query fragments of row q16 (rows past R reuse row 0; never stored):
  // k-step s, lane group g holds head-dim elements 32 s + 8 g .. +8
  bf16x8_t qf[C::NSTEP];
  auto load_q = [&]() {
    const int rc = q16 < a.rows && q16 / a.g < qn ? q16 : 0;
    const int t = rc / a.g;
    const int hl = rc - t * a.g;
    const size_t qrow = (size_t)(qb + t) * a.hq + h_kv * a.g + hl;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + qrow * D;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * s + 8 * g);
  };

  // stage m < npre: keys kbeg + 16 m .. +15, one aligned block of one page;
  // stage npre (last split only): the draft_len <= 16 draft keys.  A stage
  // m >= nst is a placeholder: every lane loads the first 16 bytes of the
  // query block (one cached line, no HBM traffic), so that every pass of
  // the stage loop issues the same loads and the compiler's wait counts stay
  // exact up to the last stage.
  auto issue = [&](int m, u32x4_t (&kd)[NLD], u32x4_t (&vd)[NLD]) {
    const int k0 = kbeg + 16 * m;
    const char* kb;
    const char* vb;
    int last;
    uint32_t stride = slot_stride;
    uint32_t lane_off = 16u * (uint32_t)pos;
    if (m < npre) {
      const uint32_t pg = (uint32_t)ptab[k0 >> ps_shift];
      const size_t base = (size_t)pg * page_bytes + (size_t)(k0 & ps_mask) * slot_stride + head_off;
      kb = kpool + base;
      vb = vpool + base;
      last = kend - 1 - k0;
    } else if (m < nst) {
      kb = reinterpret_cast<const char*>(a.k_ext) + ext_off;
      vb = reinterpret_cast<const char*>(a.v_ext) + ext_off;
      last = qn - 1;
    } else {
      kb = vb = reinterpret_cast<const char*>(a.q);
      last = 0;
      stride = 0;
      lane_off = 0;
    }
    uint32_t vo[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int key = C::RPI * j + rr;
      vo[j] = (uint32_t)(key < last ? key : last) * stride + lane_off;
    }
#pragma unroll
    for (int j = 0; j < NLD; ++j) kd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + vo[j]));
#pragma unroll
    for (int j = 0; j < NLD; ++j) vd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + vo[j]));
    // keep the stages' loads in issue order (the wait counts rely on it)
    __builtin_amdgcn_sched_barrier(0);
  };

  float m_run = kNegBig;
  float l_run = 0.f;
  f32x4_t o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float c = a.scale_log2;

  // the stage's K and V rows (register set) -> this wave's LDS tiles
  auto put = [&](const u32x4_t (&kd)[NLD], const u32x4_t (&vd)[NLD], char* kt, char* vt) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int key = C::RPI * j + rr;
      put_chunk<KDT, C::TCPR>(kt + key * C::TROWB, pos, C::fk(key), kd[j]);
      put_chunk<KDT, C::TCPR>(vt + key * C::TROWB, pos, C::fv(key), vd[j]);
    }
  };

  auto math = [&](int n, const char* kt, const char* vt) {
    const int k0 = kbeg + 16 * n;  // prefix stages only
    // ---- S^T (16 keys x 16 rows): lane (q16, g) gets keys 4g .. 4g+3 of row q16
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
    const char* krow = kt + q16 * C::TROWB;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) {
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((4 * s + g) ^ C::fk(q16)));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc, 0, 0, 0);
    }
    // ---- online softmax of the stage (prefix keys past kend, and draft keys
    // after the row's own draft position, are masked)
    const bool draft = n >= npre;
    const int lim = !draft ? kend - k0 : trow + 1;
    float mr = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = sc[e];
      bool hide;
      if constexpr (TREE) hide = draft ? !((dvis >> e) & 1u) : (4 * g + e >= lim);
      else hide = 4 * g + e >= lim;
      if (hide) x = -__builtin_inff();
      sc[e] = x;
      mr = fmaxf(mr, x);
    }
    mr = max_xor32(max_xor16(mr));  // the row's four lane groups
    const float mx = mr * c;
    const bool grow = mx > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mn = grow ? mx : m_run;
      const float al = fast_exp2(m_run - mn);
      l_run *= al;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= al;
      m_run = mn;
    }
    float p4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p4[e] = fast_exp2(__builtin_fmaf(sc[e], c, -m_run));
    l_run += (p4[0] + p4[1]) + (p4[2] + p4[3]);
    const u32x2_t pk = {pack_bf16x2(p4[0], p4[1]), pack_bf16x2(p4[2], p4[3])};
    const s16x4_t pt = __builtin_bit_cast(s16x4_t, pk);
    // ---- O^T += V^T P^T: lane (d, g) reads V rows 4g .. 4g+3 of column d transposed
    const int sp = q16 >> 2;
    const int av = q16 & 3;
    const int vr = 4 * g + sp;
    const char* vsrc = vt + vr * C::TROWB + 8 * (av & 1);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int chunk = 2 * db + (av >> 1);
      const s16x4_t vf =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16(PR_LDS_PTR(s16x4_t, vsrc + 16 * (chunk ^ C::fv(vr))));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pt, o[db], 0, 0, 0);
    }
  };

  // Stage n lives in register set n % NB.  As soon as its rows are in LDS the
  // set is reloaded with stage n + NB, before any arithmetic on stage n, so
  // that the score and softmax latency never delays a load.
  u32x4_t kr[NB][NLD], vr[NB][NLD];
  load_q();
#pragma unroll
  for (int p = 0; p < NB; ++p) issue(p, kr[p], vr[p]);
  // Retire the query loads (the oldest ones) before the stage loop: a query
  // load still pending at the loop entry would make the compiler's wait
  // counts inside the loop drain the ring on every pass.
#pragma unroll
  for (int s = 0; s < C::NSTEP; ++s) asm volatile("" ::"v"(qf[s]));
  for (int n = 0; n < nst; n += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool live = n + u < nst;
      if (live) put(kr[u], vr[u], tiles[u & 1][0], tiles[u & 1][1]);
      issue(n + u + NB, kr[u], vr[u]);
      if (live) math(n + u, tiles[u & 1][0], tiles[u & 1][1]);
    }
  }

  // ---- merge the waves' results in LDS (each wave writes into its own tile
  // area, so only the final barrier orders them), then write the split's
  // partial result: O_s = acc / l, LSE_s = M + log2 l (log2 domain)
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  if constexpr (W == 1) {
    if (q16 < a.rows) {
      const bool empty = !(lt > 0.f);
      const float inv = empty ? 0.f : 1.0f / lt;
      const size_t prow = (((size_t)b * a.hkv + h_kv) * a.n_splits + it.split) * a.rows + q16;
      __bf16* po = reinterpret_cast<__bf16*>(a.part_o) + prow * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const f32x4_t r = o[db] * inv;
        *reinterpret_cast<u32x2_t*>(po + 16 * db + 4 * g) = u32x2_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      }
      if (g == 0) a.part_lse[prow] = empty ? -__builtin_inff() : m_run + fast_log2(lt);
    }
  } else {
    float* mo = reinterpret_cast<float*>(&tiles[0][0][0]);  // [16][D]
    float* mm = mo + 16 * D;                                  // [16] running maxima
    float* ml = mm + 16;                                      // [16] sums
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) *reinterpret_cast<f32x4_t*>(mo + q16 * D + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      mm[q16] = m_run;
      ml[q16] = lt;
    }
    __syncthreads();
    // thread t of the workgroup: row t / (4 W / ... ) -- 16 rows x D columns
    // in float4 pieces, spread over all 64 W threads
    constexpr int PIECES = 16 * D / 4;
    constexpr int STRIDE = 64 * W;
    const int stride_w = 2 * 2 * C::TILE / 4;  // floats between two waves' areas
    const float* base = reinterpret_cast<const float*>(&tiles_all[0][0][0][0]);
    for (int pc = threadIdx.x; pc < PIECES; pc += STRIDE) {
      const int r = pc / (D / 4);
      const int c4 = pc - r * (D / 4);
      if (r >= a.rows) continue;
      // every wave's values are read first and combined with selects: a
      // branch per wave kept each read one LDS round trip behind the last
      float mw[W], lw[W];
      f32x4_t xw[W];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        mw[w] = base[w * stride_w + 16 * D + r];
        lw[w] = base[w * stride_w + 16 * D + 16 + r];
        xw[w] = *reinterpret_cast<const f32x4_t*>(base + w * stride_w + r * D + 4 * c4);
      }
      float mx = kNegBig;
#pragma unroll
      for (int w = 0; w < W; ++w) mx = fmaxf(mx, mw[w]);
      float lsum = 0.f;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < W; ++w) {
        // a wave that saw no key has l = 0 and a zero accumulator
        const float sc = lw[w] > 0.f ? fast_exp2(mw[w] - mx) : 0.f;
        lsum += lw[w] * sc;
        acc += sc * xw[w];
      }
      const bool empty = !(lsum > 0.f);
      const float inv = empty ? 0.f : 1.0f / lsum;
      const size_t prow = (((size_t)b * a.hkv + h_kv) * a.n_splits + it.split) * a.rows + r;
      const f32x4_t ov = acc * inv;
      *reinterpret_cast<u32x2_t*>(reinterpret_cast<__bf16*>(a.part_o) + prow * D + 4 * c4) =
          u32x2_t{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
      if (c4 == 0) a.part_lse[prow] = empty ? -__builtin_inff() : mx + fast_log2(lsum);
    }
  }
}

// Merge of the splits' partial results, one wave per (stacked row, 64-column
// slice): O = v_scale * sum_s w_s O_s / sum_s w_s, LSE = ln 2 * (M + log2
// sum_s w_s) with w_s = exp2(LSE_s - M), M = max_s LSE_s (empty splits have
// LSE_s = -inf and weight 0).  Lane l takes columns 4 (l % 16) .. +3 of the
// slice in the splits s = l / 16 (mod 4): one 16-byte load per split, up to
// 16 splits in flight per lane; the four split groups are then summed across
// lanes.  Lane s holds split s's log-sum-exp (n_splits <= 64).  The split
// passes that feed it (register and wide streaming) store their partial O in
// bf16 (8-byte loads here); the queries, and so O, are bf16.
template <int D>
__global__ __launch_bounds__(256) void paged_merge_kernel(PagedArgs a) {
  constexpr int NCH = D / 64;
  constexpr int MB = 16;  // splits per lane (4 groups x 16 = 64 splits at most)
  const int gw = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * 256 + threadIdx.x) >> 6));
  const int lane = threadIdx.x & 63;
  if (gw >= a.batch * a.hkv * a.rows * NCH) return;
  const int ch = gw % NCH;
  const int rw = gw / NCH;
  const int r = rw % a.rows;
  const int h_kv = (rw / a.rows) % a.hkv;
  const int b = rw / (a.rows * a.hkv);
  const int t = r / a.g;
  const int hl = r - t * a.g;
  if (t >= draft_count(a.qo_indptr, b, a.draft_len)) return;  // past the request's draft rows
  const size_t qrow = (size_t)(draft_base(a.qo_indptr, b, a.draft_len) + t) * a.hq + h_kv * a.g + hl;
  const size_t prow0 = (((size_t)b * a.hkv + h_kv) * a.n_splits) * a.rows + r;
  const size_t sstride = (size_t)a.rows * D;
  const int ns = a.n_splits;
  const int c = lane & 15;
  const int gi = lane >> 4;
  const size_t po = prow0 * D + 64 * ch + 4 * c;  // element offset of split 0

  const float ls = lane < ns ? a.part_lse[prow0 + (size_t)lane * a.rows] : -__builtin_inff();
  f32x4_t x[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int sp = gi + 4 * u;
    if (sp < ns) {
      const u32x2_t h = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const __bf16*>(a.part_o) + po +
                                                         (size_t)sp * sstride);
      x[u] = f32x4_t{__builtin_bit_cast(float, h[0] << 16), __builtin_bit_cast(float, h[0] & 0xffff0000u),
                     __builtin_bit_cast(float, h[1] << 16), __builtin_bit_cast(float, h[1] & 0xffff0000u)};
    }
  }
  const float mt = wave_max(ls);
  const float w = ls == -__builtin_inff() ? 0.f : fast_exp2(ls - mt);
  const float wsum = wave_sum(w);
  // an empty split (weight 0) holds zeros; its data is never multiplied
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int sp = gi + 4 * u;
    const float ws = __shfl(w, sp < 64 ? sp : 63);
    if (sp < ns && ws != 0.f) acc += ws * x[u];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  if (gi == 0) {
    const float sc = wsum > 0.f ? a.v_scale / wsum : 0.f;
    const size_t oi = qrow * D + 64 * ch + 4 * c;
    const u32x2_t v = {pack_bf16x2(acc[0] * sc, acc[1] * sc), pack_bf16x2(acc[2] * sc, acc[3] * sc)};
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<__bf16*>(a.o) + oi) = v;
  }
  if (ch == 0 && lane == 0) a.lse[qrow] = wsum > 0.f ? (mt + fast_log2(wsum)) * kLn2 : -__builtin_inff();
}

template <int D, int KDT>
int launch_t(const PagedArgs& a, int64_t n_blocks, hipStream_t s) {
  constexpr int OCC = D <= 128 ? 2 : 1;
  constexpr int W = reg_waves(D);
  if (a.draft_mask)
    hipLaunchKernelGGL((paged_reg_kernel<D, KDT, OCC, W, true>), dim3((unsigned)n_blocks), dim3(64 * W), 0, s, a);
  else
    hipLaunchKernelGGL((paged_reg_kernel<D, KDT, OCC, W, false>), dim3((unsigned)n_blocks), dim3(64 * W), 0, s, a);
  return (int)hipGetLastError();
}

template <int D>
int launch_merge_t(const PagedArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.batch * a.hkv * a.rows * (D / 64);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks == 0) return 0;
  hipLaunchKernelGGL((paged_merge_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_paged_merge(const PagedArgs& a, int d, int q_dtype, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.n_splits > 64 || q_dtype != DT_BF16 || !a.part_bf16) return (int)hipErrorInvalidValue;
  switch (d) {
    case 64: return launch_merge_t<64>(a, s);
    case 128: return launch_merge_t<128>(a, s);
    case 256: return launch_merge_t<256>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

int launch_paged_reg(const PagedArgs& a, int d, int kv_dtype, int64_t n_blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.rows > 16 || a.draft_len > 16 || a.page_size < 16 || (a.page_size & (a.page_size - 1)) != 0 ||
      a.split_len % 16 != 0 || a.n_splits > 64)
    return (int)hipErrorInvalidValue;
  if (kv_dtype == DT_BF16) {
    switch (d) {
      case 64: return launch_t<64, DT_BF16>(a, n_blocks, s);
      case 128: return launch_t<128, DT_BF16>(a, n_blocks, s);
      case 256: return launch_t<256, DT_BF16>(a, n_blocks, s);
    }
  } else if (kv_dtype == DT_FP8) {
    switch (d) {
      case 64: return launch_t<64, DT_FP8>(a, n_blocks, s);
      case 128: return launch_t<128, DT_FP8>(a, n_blocks, s);
      case 256: return launch_t<256, DT_FP8>(a, n_blocks, s);
    }
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace psattn
