// psattn_widestream.hip -- split-KV verify pass for 17..64 stacked query rows
// (draft_len * G) over a paged bf16 or OCP fp8 e4m3fn KV cache, gfx950.
//
// sglang PR #27382 ("实现拆解", implementation breakdown) splits the verify
// path into a first stage that walks the long paged prefix in splits and
// writes one partial (O, LSE) per split, and a second stage that merges them
// with the small causal draft block.  With up to 64 stacked rows a key is
// worth 128 flop per fp8 byte, so this stage has to keep the matrix cores,
// the fp8 conversion and the HBM stream busy at once:
//
//  * one workgroup of 8 waves (two per SIMD) per (request, kv head, split),
//    one workgroup per CU.  The split is walked in 64-key superstages; wave w
//    loads the aligned 8-key block w of each superstage (one page, so a
//    scalar base) with whole-row coalesced 16-byte vector loads into a ring
//    of NB register sets, refilled as soon as a set is in LDS;
//  * each wave converts its block to bf16 once (fp8 codes exactly) into a
//    shared, double-buffered LDS superstage tile, one superstage ahead of
//    the arithmetic (so LDS writes overlap the MFMA work); one barrier per
//    superstage.  With fp8 K at D = 128 or 256 the K rows stay fp8 in LDS
//    (half the bytes written and read, no conversion) and the scores run on
//    v_mfma_f32_16x16x128_f8f6f4 against the query rows split into two fp8
//    terms (below);
//  * wave (rq, kh) computes stacked rows 16 rq .. 16 rq + 15 against keys
//    32 kh .. 32 kh + 31 of the superstage with v_mfma_f32_16x16x32_bf16:
//    S^T = K Q^T (K rows from LDS, Q^T fragments in registers), online
//    softmax in the log2 domain with lazy rescaling, O^T += V^T P^T with V^T
//    read by ds_read_b64_tr_b16 and P^T taken from the score registers.  The
//    two key halves keep separate softmax states and are merged through LDS
//    at the end.  Small per-wave blocks keep the registers at two waves per
//    SIMD, which is what hides the HBM latency; the price is that every K/V
//    element is read from LDS four times (LDS reads are cheap on this part);
//  * the last split of each (request, kv head) also runs the causal draft
//    block as one more superstage (draft row j sees draft keys 0..j);
//  * k_scale is folded into the logit scale; v_scale is applied by the merge;
//  * the split's partial O is stored in bf16 (its LSE in fp32): half the
//    bytes of the partials written here and read back by the merge.
//
// Contraction order of O^T += V^T P^T: position 8 g + 4 j + e of the 32 keys
// of a wave (lane group g, score block j, element e) is key 16 j + 4 g + e,
// which is where the score MFMA leaves it; V^T is read in that order.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace psattn {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

#define PW_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kWideWaves = 8;

template <int D, int KDT>
struct WCfg {
  static constexpr int ES = Elem<KDT>::size;
  static constexpr int ROWB = D * ES;    // global bytes of one key row of one kv head
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per global row
  static constexpr int RPI = 64 / CPR;   // rows covered by one wave-wide load
  static constexpr int NLK = (8 + RPI - 1) / RPI;  // loads per lane for the wave's 8 K rows (same for V)
  static constexpr int TROWB = 2 * D;    // LDS row bytes (bf16)
  static constexpr int TCPR = TROWB / 16;
  static constexpr int TILE = 64 * TROWB;  // one 64-key K (or V) superstage tile
  static constexpr int NSTEP = D / 32;     // k-steps of the score product
  static constexpr int NDB = D / 16;       // 16-column output blocks
  // register sets in the ring: about 128 bytes (32 VGPRs) of K/V per lane,
  // at most 4 sets (two waves per SIMD leave no room for more)
  static constexpr int NBR = 128 / (2 * NLK * 16);
  static constexpr int NB = NBR >= 4 ? 4 : (NBR >= 1 ? NBR : 1);
  static constexpr int UNR = NB >= 2 ? NB : 2;  // superstages per pass of the loop
  static_assert(CPR <= 64 && NB >= 1, "shape");
  __device__ static constexpr int fk(int r) { return r & (TCPR - 1); }
  __device__ static constexpr int fv(int r) { return (2 * r) & (TCPR - 1); }
  // fp8 K with D a multiple of 128: K stays fp8 in LDS (rows of D bytes) and
  // the scores run on v_mfma_f32_16x16x128_f8f6f4 against the query split
  // into two fp8 terms
  static constexpr bool F8S = KDT == DT_FP8 && D % 128 == 0;
  static constexpr int KROWB = F8S ? D : TROWB;  // LDS bytes of a K row
  static constexpr int KCPR = KROWB / 16;
  static constexpr int NSD = D / 128;            // 128-deep k-steps of the fp8 score product
  __device__ static constexpr int fk8(int r) { return r & (KCPR - 1); }
};

typedef int i8v_t __attribute__((ext_vector_type(8)));

// gfx950 fp8 forms, kept in device functions (the host pass of a kernel body
// that names them directly drops the kernel)
// fp8 (e4m3) codes of x0..x3 in bytes 0..3, and their decoded values
__device__ __forceinline__ int fp8x4_split(float x0, float x1, float x2, float x3, float& h0, float& h1, float& h2,
                                           float& h3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  h0 = __builtin_amdgcn_cvt_f32_fp8(w, 0);
  h1 = __builtin_amdgcn_cvt_f32_fp8(w, 1);
  h2 = __builtin_amdgcn_cvt_f32_fp8(w, 2);
  h3 = __builtin_amdgcn_cvt_f32_fp8(w, 3);
  return w;
}
// 16 x 16 x 128 fp8 x fp8 product, unscaled
__device__ __forceinline__ f32x4_t mfma_fp8_16x16x128(const i8v_t a, const i8v_t b, const f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// the exponent e of x = f 2^e, f in [1/2, 1)
__device__ __forceinline__ int frexp_exponent(float x) { return __builtin_amdgcn_frexp_expf(x); }

// 16 bytes of a global row (chunk pos) -> the row's LDS tile slot(s), as bf16
template <int KDT>
__device__ __forceinline__ void wput(char* trow, int pos, int f, const u32x4_t x) {
  if constexpr (KDT == DT_BF16) {
    *reinterpret_cast<u32x4_t*>(trow + 16 * (pos ^ f)) = x;
  } else {
    u32x4_t lo, hi;
    fp8x16_to_bf16(x, lo, hi);
    *reinterpret_cast<u32x4_t*>(trow + 16 * ((2 * pos) ^ f)) = lo;
    *reinterpret_cast<u32x4_t*>(trow + 16 * ((2 * pos + 1) ^ f)) = hi;
  }
}

// TREE: the draft block follows the request's draft mask (a compile-time
// variant, so that the causal kernel keeps its own code)
template <int D, int KDT, bool TREE>
__global__ __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(2)))
void paged_wide_kernel(PagedArgs a) {
  using C = WCfg<D, KDT>;
  constexpr int NB = C::NB;
  constexpr int NLK = C::NLK;
  // [buffer][K, V] superstage tiles; reused at the end for the merge
  __shared__ __attribute__((aligned(16))) char tiles[2][2][C::TILE];

  const Item it = paged_item(blockIdx.x, a.hkv, a.n_splits, a.split_len, a.draft_len, a.prefix_lens);
  const int b = it.seg;
  const int h_kv = it.h_kv;
  const int qb = draft_base(a.qo_indptr, b, a.draft_len);  // the request's first draft row
  const int qn = draft_count(a.qo_indptr, b, a.draft_len);  // and its number of draft rows
  if (qn <= 0) return;                                       // a request without draft rows
  const int kbeg = it.r0_begin;
  const int kend = it.r0_end;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int rq = wave & 3;   // row quarter
  const int kh = wave >> 2;  // key half of each superstage
  const int lane = threadIdx.x & 63;
  const int q16 = lane & 15;
  const int g = lane >> 4;
  const int pos = lane % C::CPR;  // load layout: chunk pos of row RPI j + rr
  const int rr = lane / C::CPR;
  const int ps_shift = __builtin_ctz((unsigned)a.page_size);
  const int ps_mask = a.page_size - 1;
  typedef const __attribute__((address_space(4))) int32_t* ctab_t;
  const ctab_t ptab = reinterpret_cast<ctab_t>(reinterpret_cast<uintptr_t>(a.kv_indices + a.kv_indptr[b]));
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const uint32_t slot_stride = (uint32_t)a.hkv * C::ROWB;
  const size_t page_bytes = (size_t)slot_stride << ps_shift;
  const size_t head_off = (size_t)h_kv * C::ROWB;
  const int npre = (kend - kbeg + 63) >> 6;
  const int nst = npre + (it.split == a.n_splits - 1 ? 1 : 0);
  const size_t ext_off = ((size_t)qb * a.hkv + h_kv) * C::ROWB;
  const int myrow = 16 * rq + q16;  // stacked row of this lane's scores
  const int trow = (myrow < a.rows ? myrow : 0) / a.g;
  // draft keys 32 kh + 16 j + 4 g + e (j = 0, 1; e = 0..3) this lane's row
  // sees: its draft-mask row, or the causal chain (keys 0 .. trow)
  uint32_t dvis = 0;
  if constexpr (TREE) {
    const uint8_t* mrow = a.draft_mask + ((size_t)b * a.draft_len + trow) * a.draft_len;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 32 * kh + 16 * j + 4 * g + e;
        const bool v = key < qn && mrow[key] != 0;
        dvis |= (v ? 1u : 0u) << (4 * j + e);
      }
    asm volatile("" ::"v"(dvis));  // retired here, before the stage ring
  }

  // ---- query fragments (B operand of S^T = K Q^T): row 16 rq + q16,
  // k-step s, lane group g holds head-dim elements 32 s + 8 g .. +8
  bf16x8_t qf[C::F8S ? 1 : C::NSTEP];
  // F8S: Q^T as the B operand of the fp8 product, k-step sd, lane group g
  // holding head-dim elements 128 sd + 32 g .. +32, each row scaled by a power
  // of two 2^qe that puts its largest magnitude in [128, 256) and split into
  // hi = fp8(x) and lo = fp8(x - hi), which sum to x exactly wherever
  // |x| >= 1/4 (a bf16 value has 8 significant bits, each fp8 term 4) and to
  // within 2^-10 below; cq = the logit scale over 2^qe.
  i8v_t qh[C::F8S ? C::NSD : 1], ql[C::F8S ? C::NSD : 1];
  float cq = a.scale_log2;
  // F8S: the query row's 16-byte pieces, fetched before the first
  // superstage's loads are issued and split after them, so that the split
  // waits only for the query and the K/V latency runs under it
  u32x4_t qraw[C::F8S ? C::NSD : 1][4];
  auto load_q = [&]() {
    const int rc = myrow < a.rows && myrow / a.g < qn ? myrow : 0;
    const int t = rc / a.g;
    const int hl = rc - t * a.g;
    const size_t qrow = (size_t)(qb + t) * a.hq + h_kv * a.g + hl;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + qrow * D;
    if constexpr (C::F8S) {
#pragma unroll
      for (int sd = 0; sd < C::NSD; ++sd)
#pragma unroll
        for (int u = 0; u < 4; ++u) qraw[sd][u] = *reinterpret_cast<const u32x4_t*>(qp + 128 * sd + 32 * g + 8 * u);
    } else {
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * s + 8 * g);
    }
  };
  auto split_q = [&]() {
    if constexpr (C::F8S) {
      float x[C::NSD][32];
      float am = 0.f;
#pragma unroll
      for (int sd = 0; sd < C::NSD; ++sd)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // bf16 element e: the high or low half of dword e / 2, as fp32 bits
            const uint32_t w = qraw[sd][u][e >> 1];
            x[sd][8 * u + e] = __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
            am = fmaxf(am, fabsf(x[sd][8 * u + e]));
          }
      am = fmaxf(am, __shfl_xor(am, 16));
      am = fmaxf(am, __shfl_xor(am, 32));
      // am = f 2^ex with f in [1/2, 1): scale by 2^(8 - ex)
      const int qe = am > 0.f ? 8 - frexp_exponent(am) : 0;
      cq = a.scale_log2 * __builtin_ldexpf(1.0f, -qe);
#pragma unroll
      for (int sd = 0; sd < C::NSD; ++sd)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float x0 = __builtin_ldexpf(x[sd][4 * w], qe);
          const float x1 = __builtin_ldexpf(x[sd][4 * w + 1], qe);
          const float x2 = __builtin_ldexpf(x[sd][4 * w + 2], qe);
          const float x3 = __builtin_ldexpf(x[sd][4 * w + 3], qe);
          float h0, h1, h2, h3, l0, l1, l2, l3;
          qh[sd][w] = fp8x4_split(x0, x1, x2, x3, h0, h1, h2, h3);
          ql[sd][w] = fp8x4_split(x0 - h0, x1 - h1, x2 - h2, x3 - h3, l0, l1, l2, l3);
        }
    }
  };

  // superstage m: this wave's aligned 8-key block (keys k0 + 8 wave ..);
  // m == npre (last split): the draft block; m >= nst: placeholder loads of
  // one cached query chunk, so that every pass issues the same loads
  auto issue = [&](int m, u32x4_t (&kd)[NLK], u32x4_t (&vd)[NLK]) {
    const char* kb;
    const char* vb;
    int lastr;  // last valid row of the block
    uint32_t stride = slot_stride;
    uint32_t lane_off = 16u * (uint32_t)pos;
    if (m < npre) {
      const int kb0 = kbeg + 64 * m + 8 * wave;
      const int klast = kend - 1;
      const int kbe = kb0 <= klast ? kb0 : (klast & ~7);
      const uint32_t pg = (uint32_t)ptab[kbe >> ps_shift];
      const size_t base = (size_t)pg * page_bytes + (size_t)(kbe & ps_mask) * slot_stride + head_off;
      kb = kpool + base;
      vb = vpool + base;
      lastr = klast - kbe;
    } else if (m < nst) {
      const size_t base = ext_off + (size_t)(8 * wave) * slot_stride;
      kb = reinterpret_cast<const char*>(a.k_ext) + base;
      vb = reinterpret_cast<const char*>(a.v_ext) + base;
      lastr = qn - 1 - 8 * wave;
      if (lastr < 0) {  // no draft rows in this block: reread the first one
        kb = reinterpret_cast<const char*>(a.k_ext) + ext_off;
        vb = reinterpret_cast<const char*>(a.v_ext) + ext_off;
        lastr = 0;
      }
    } else {
      kb = vb = reinterpret_cast<const char*>(a.q);
      lastr = 0;
      stride = 0;
      lane_off = 0;
    }
    uint32_t vo[NLK];
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      int r = C::RPI * j + rr;
      r = r < 8 ? r : r - 8;  // lanes past the 8 rows (short rows) duplicate
      vo[j] = (uint32_t)(r < lastr ? r : lastr) * stride + lane_off;
    }
#pragma unroll
    for (int j = 0; j < NLK; ++j) kd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + vo[j]));
#pragma unroll
    for (int j = 0; j < NLK; ++j) vd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + vo[j]));
    __builtin_amdgcn_sched_barrier(0);
  };

  auto put = [&](const u32x4_t (&kd)[NLK], const u32x4_t (&vd)[NLK], char* kt, char* vt) {
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const int r = C::RPI * j + rr;
      if (C::RPI * NLK <= 8 || r < 8) {
        const int row = 8 * wave + r;
        if constexpr (C::F8S)
          *reinterpret_cast<u32x4_t*>(kt + row * C::KROWB + 16 * (pos ^ C::fk8(row))) = kd[j];
        else
          wput<KDT>(kt + row * C::TROWB, pos, C::fk(row), kd[j]);
        wput<KDT>(vt + row * C::TROWB, pos, C::fv(row), vd[j]);
      }
    }
  };

  float m_run = kNegBig;
  float l_run = 0.f;
  f32x4_t o[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto math = [&](int n, const char* kt, const char* vt) {
    const float c = cq;  // logit scale (log2 domain) of this lane's row
    // keys 32 kh .. 32 kh + 31 of superstage n; lim = keys of the half that
    // this lane's row may see
    const int kofs = 32 * kh;
    const bool draft = n >= npre;
    const int lim = !draft ? kend - (kbeg + 64 * n) - kofs : (trow + 1) - kofs;
    // ---- S^T blocks j = 0, 1 (16 keys x 16 rows): lane (q16, g) gets keys
    // 16 j + 4 g .. +3 of row q16
    f32x4_t sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int kr = kofs + 16 * j + q16;
      if constexpr (C::F8S) {
        // A operand: key row kr, head-dim bytes 128 sd + 32 g .. +32 (two chunks)
        const char* krow = kt + kr * C::KROWB;
#pragma unroll
        for (int sd = 0; sd < C::NSD; ++sd) {
          const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(krow + 16 * ((8 * sd + 2 * g) ^ C::fk8(kr)));
          const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(krow + 16 * ((8 * sd + 2 * g + 1) ^ C::fk8(kr)));
          const i8v_t kf = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3], (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
          sc[j] = mfma_fp8_16x16x128(kf, qh[sd], sc[j]);
          sc[j] = mfma_fp8_16x16x128(kf, ql[sd], sc[j]);
        }
      } else {
        const char* krow = kt + kr * C::TROWB;
#pragma unroll
        for (int s = 0; s < C::NSTEP; ++s) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((4 * s + g) ^ C::fk(kr)));
          sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc[j], 0, 0, 0);
        }
      }
    }
    float mr = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = sc[j][e];
        bool hide;
        if constexpr (TREE) hide = draft ? !((dvis >> (4 * j + e)) & 1u) : (16 * j + 4 * g + e >= lim);
        else hide = 16 * j + 4 * g + e >= lim;
        if (hide) x = -__builtin_inff();
        sc[j][e] = x;
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
    bf16x8_t pt;  // P^T position 8 g + 4 j + e
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(__builtin_fmaf(sc[j][e], c, -m_run));
        pt[4 * j + e] = (__bf16)p;
        psum += p;
      }
    l_run += psum;
    // ---- O^T += V^T P^T: lane (d, g) reads V rows 16 j + 4 g .. +3 of
    // column d transposed (in-group source lane ap + 4 sp addresses row
    // 16 j + 4 g + sp, columns 4 ap ..)
    const int sp = q16 >> 2;
    const int ap = q16 & 3;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      s16x4_t vv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = kofs + 16 * j + 4 * g + sp;
        const int chunk = 2 * db + (ap >> 1);
        vv[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            PW_LDS_PTR(s16x4_t, vt + row * C::TROWB + 16 * (chunk ^ C::fv(row)) + 8 * (ap & 1)));
      }
      const s16x8_t v8 = {vv[0][0], vv[0][1], vv[0][2], vv[0][3], vv[1][0], vv[1][1], vv[1][2], vv[1][3]};
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v8), pt, o[db], 0, 0, 0);
    }
  };

  // Software pipeline over superstages: pass n converts and writes
  // superstage n + 1 into one LDS buffer while the arithmetic of superstage n
  // reads the other, then one barrier publishes n + 1 and retires n.  The
  // register set of n + 1 is refilled with superstage n + 1 + NB right after
  // its rows are in LDS.
  u32x4_t kr[NB][NLK], vr[NB][NLK];
  load_q();
#pragma unroll
  for (int p = 0; p < NB; ++p) issue(p, kr[p], vr[p]);
  // retire the query loads (the oldest) before the loop, so that the
  // compiler's wait counts inside it stay exact (the fp8 split consumes them)
  split_q();
#pragma unroll
  for (int s = 0; s < (C::F8S ? 0 : C::NSTEP); ++s) asm volatile("" ::"v"(qf[s]));
  if (nst > 0) put(kr[0], vr[0], tiles[0][0], tiles[0][1]);
  issue(NB, kr[0], vr[0]);
  __syncthreads();
  for (int n = 0; n < nst; n += C::UNR) {
    // UNR superstages per pass, so that the register set ((n + 1) % NB) and
    // the LDS buffers ((n + 1) % 2, n % 2) are compile-time constants
#pragma unroll
    for (int u = 0; u < C::UNR; ++u) {
      const int nx = n + u + 1;  // superstage written in this step
      if (nx < nst) put(kr[(u + 1) % NB], vr[(u + 1) % NB], tiles[(u + 1) & 1][0], tiles[(u + 1) & 1][1]);
      issue(nx + NB, kr[(u + 1) % NB], vr[(u + 1) % NB]);
      if (n + u < nst) math(n + u, tiles[u & 1][0], tiles[u & 1][1]);
      __syncthreads();
    }
  }

  // ---- merge the two key halves of each row quarter: the kh = 1 waves hand
  // their state over through LDS, the kh = 0 waves combine it with their own
  // registers and write the split's partial result:
  // O_s = acc / l, LSE_s = M + log2 l (log2 domain)
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  __syncthreads();  // every wave is done with the tiles
  float* mo = reinterpret_cast<float*>(&tiles[0][0][0]);  // [64 rows][D]
  float* mm = mo + 64 * D;                                  // [64]
  float* ml = mm + 64;                                      // [64]
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
      *reinterpret_cast<f32x4_t*>(mo + myrow * D + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      mm[myrow] = m_run;
      ml[myrow] = lt;
    }
  }
  __syncthreads();
  if (kh == 0 && myrow < a.rows) {
    const float m1 = mm[myrow];
    const float l1 = ml[myrow];
    const float mx = fmaxf(m_run, m1);
    const float s0 = lt > 0.f ? fast_exp2(m_run - mx) : 0.f;
    const float s1 = l1 > 0.f ? fast_exp2(m1 - mx) : 0.f;
    const float lsum = lt * s0 + l1 * s1;
    const bool empty = !(lsum > 0.f);
    const float inv = empty ? 0.f : 1.0f / lsum;
    const float w0 = s0 * inv, w1 = s1 * inv;
    const size_t prow = (((size_t)b * a.hkv + h_kv) * a.n_splits + it.split) * a.rows + myrow;
    // the partial O in bf16: half the bytes written here and read by the merge
    __bf16* po = reinterpret_cast<__bf16*>(a.part_o) + prow * D;
    // the other half's values are all read before the first store (one read
    // issued per store left each store an LDS round trip behind the last)
    f32x4_t x1s[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) x1s[db] = *reinterpret_cast<const f32x4_t*>(mo + myrow * D + 16 * db + 4 * g);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d0 = 16 * db + 4 * g;
      const f32x4_t x1 = x1s[db];
      f32x4_t r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (w0 != 0.f ? w0 * o[db][e] : 0.f) + (w1 != 0.f ? w1 * x1[e] : 0.f);
      const u32x2_t v = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      *reinterpret_cast<u32x2_t*>(po + d0) = v;
    }
    if (g == 0) a.part_lse[prow] = empty ? -__builtin_inff() : mx + fast_log2(lsum);
  }
}

template <int D, int KDT>
int launch_t(const PagedArgs& a, int64_t n_blocks, hipStream_t s) {
  if (a.draft_mask) {
    hipLaunchKernelGGL((paged_wide_kernel<D, KDT, true>), dim3((unsigned)n_blocks), dim3(64 * kWideWaves), 0, s, a);
    return (int)hipGetLastError();
  }
  static_assert(64 * D * 4 + 2 * 64 * 4 <= 4 * WCfg<D, KDT>::TILE, "merge area");
  hipLaunchKernelGGL((paged_wide_kernel<D, KDT, false>), dim3((unsigned)n_blocks), dim3(64 * kWideWaves), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_paged_wide(const PagedArgs& a, int d, int kv_dtype, int64_t n_blocks, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.rows > 64 || a.draft_len > 64 || a.page_size < 16 || (a.page_size & (a.page_size - 1)) != 0 ||
      a.split_len % 64 != 0 || a.n_splits > 64)
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
