// psattn_stream.hip -- split-KV prefix pass for speculative verify over a
// paged KV cache with bf16 or OCP fp8 e4m3fn K/V, gfx950.
//
// sglang PR #27382 ("实现拆解", implementation breakdown) describes the
// verify path as a first stage that walks the long paged prefix in splits,
// applies the fp8 scaling and writes one partial result per split, and a
// second stage that merges the splits by log-sum-exp together with the small
// causal draft block.  This file is the first stage, built for HBM streaming:
//
//  * workgroup = (request, kv head, split) with 4 waves; its page list is
//    copied into LDS once, so no page-id load sits on the critical path;
//  * the split is walked in 32-key stages through a 3-slot LDS ring.  Each
//    stage is copied global -> LDS with 16-byte global_load_lds_dwordx4
//    (no register staging), a quarter of the copies issued by each wave, two
//    stages ahead of the one being computed; one barrier per stage;
//  * all 4 waves read the same stage.  The R = draft_len * G stacked query
//    rows are spread over the waves as RG row groups x DS slices of the head
//    dimension: every wave computes the scores of its rows over the full
//    head dimension (so it owns complete softmax statistics) and the output
//    columns of its slice, and the workgroup needs no final merge;
//  * scores S^T = K Q^T use v_mfma_f32_16x16x32_bf16 with K rows read from
//    LDS in an order chosen so that a lane's 8 scores are 8 consecutive keys;
//    O^T += V^T P^T then takes P^T straight from the score registers and V^T
//    from the row-major V tile with the gfx950 transpose reads
//    ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (fp8);
//  * fp8 codes are converted to bf16 exactly in registers; k_scale is folded
//    into the logit scale, v_scale is applied by the combine stage;
//  * online softmax in the log2 domain with lazy rescaling: the running
//    maximum used by the exponentials only moves when a row's new maximum
//    exceeds it by more than kTau, which keeps exp2 arguments <= kTau.
//
// LDS tiles are row-major [32 keys][D * elem] with 16-byte chunks XOR-swizzled
// per row (K: chunk ^ (row % CPR); V: chunk ^ (2 row % CPR)) so that the
// score-operand reads and the transpose reads avoid bank conflicts.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace psattn {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

#define PS_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4_t r;
  r[0] = fp8x2_to_bf16x2<false>(w0);
  r[1] = fp8x2_to_bf16x2<true>(w0);
  r[2] = fp8x2_to_bf16x2<false>(w1);
  r[3] = fp8x2_to_bf16x2<true>(w1);
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int D, int KDT, int SK_, int NW_, int NS_>
struct SCfg {
  static constexpr int ES = Elem<KDT>::size;
  static constexpr int ROWB = D * ES;            // bytes of one key row (one kv head)
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int SK = SK_;                 // keys per stage (16 or 32)
  static constexpr int NW = NW_;                 // waves per workgroup
  static constexpr int TILE = SK * ROWB;         // bytes of a K (or V) stage tile
  static constexpr int TILE_DMA = TILE / 1024;   // wave-wide copies per tile
  static constexpr int PWD = 2 * TILE_DMA / NW;  // copies per wave per stage (K + V)
  static constexpr int SLOT = 2 * TILE;          // K + V
  static constexpr int NS = NS_;                 // ring depth
  static_assert(2 * TILE_DMA % NW == 0, "copies split evenly over the waves");
  __device__ static constexpr int fk(int r) { return r & (CPR - 1); }
  __device__ static constexpr int fv(int r) { return (2 * r) & (CPR - 1); }
};

// Wait until at most k stages of this wave's copies are still in flight
// (k is 0 .. KMAX and known only at run time; s_waitcnt takes an immediate).
template <int PWD, int KMAX>
__device__ __forceinline__ void wait_stages(int k) {
  static_assert(KMAX <= 7 && KMAX * PWD <= 63, "vmcnt range");
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PWD>(); break;
    case 2: if constexpr (KMAX >= 2) { wait_vmcnt<2 * PWD>(); break; } [[fallthrough]];
    case 3: if constexpr (KMAX >= 3) { wait_vmcnt<3 * PWD>(); break; } [[fallthrough]];
    case 4: if constexpr (KMAX >= 4) { wait_vmcnt<4 * PWD>(); break; } [[fallthrough]];
    case 5: if constexpr (KMAX >= 5) { wait_vmcnt<5 * PWD>(); break; } [[fallthrough]];
    case 6: if constexpr (KMAX >= 6) { wait_vmcnt<6 * PWD>(); break; } [[fallthrough]];
    default: if constexpr (KMAX >= 7) { wait_vmcnt<7 * PWD>(); break; } wait_vmcnt<0>(); break;
  }
}

// Workgroup of NW waves = RG row groups x DS head-dim slices; NQB 16-row blocks
// per wave; SK-key stages through an NS-slot ring; MAXP page-table entries.
template <int D, int KDT, int SK, int NW, int NS, int RG, int DS, int NQB, int MAXP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1)))
void paged_stream_kernel(PagedArgs a) {
  static_assert(RG * DS == NW, "waves");
  static_assert(SK == 32 || KDT == DT_BF16, "16-key stages are bf16 only");
  using C = SCfg<D, KDT, SK, NW, NS>;
  constexpr int NDB = D / 16 / DS;  // 16-column output blocks per wave
  __shared__ __attribute__((aligned(1024))) char ring[C::NS * C::SLOT];
  __shared__ int32_t ptab[MAXP];

  const Item it = paged_item(blockIdx.x, a.hkv, a.n_splits, a.split_len, a.draft_len, a.prefix_lens);
  const int b = it.seg;
  const int qbase = draft_base(a.qo_indptr, b, a.draft_len);  // the request's first draft row
  const int qn = draft_count(a.qo_indptr, b, a.draft_len);    // and its number of draft rows
  if (qn <= 0) return;                                         // a request without draft rows
  const int h_kv = it.h_kv;
  const int kbeg = it.r0_begin;
  const int kend = it.r0_end;
  const int tid = threadIdx.x;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / DS;
  const int ds = wave - rg * DS;
  const int lane = tid & 63;
  const int q16 = lane & 15;
  const int g = lane >> 4;
  const int ps = a.page_size;  // a power of two on this path
  const int ps_shift = __builtin_ctz((unsigned)ps);

  // ---- the split's page list -> LDS
  const int pfirst = kbeg >> ps_shift;
  const int np = kend > kbeg ? ((kend - 1) >> ps_shift) - pfirst + 1 : 0;
  {
    const int32_t* src = a.kv_indices + a.kv_indptr[b] + pfirst;
    for (int i = tid; i < np; i += NW * 64) ptab[i] = src[i];
  }

  // ---- query fragments: row 16 (rg NQB + qb) + q16, d = 32 s + 8 g .. +8
  bf16x8_t qf[NQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = (rg * NQB + qb) * 16 + q16;
    const int rc = r < a.rows && r / a.g < qn ? r : 0;
    const int t = rc / a.g;
    const int hl = rc - t * a.g;
    const size_t qrow = (size_t)(qbase + t) * a.hq + h_kv * a.g + hl;
    const u32x4_t* qp =
        reinterpret_cast<const u32x4_t*>(reinterpret_cast<const __bf16*>(a.q) + qrow * D + 8 * g);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[qb][s] = __builtin_bit_cast(bf16x8_t, qp[4 * s]);
  }
  // Retire the query loads here: otherwise the compiler waits for them at
  // their first use inside the stage loop, where a vmcnt wait would also
  // drain the copies of the next stages.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) asm volatile("" ::"v"(qf[qb][s]));

  float m[NQB], l[NQB];
  f32x4_t o[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = kNegBig;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[qb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  __syncthreads();  // page list visible

  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const int nst = (kend - kbeg + C::SK - 1) / C::SK;
  const float c = a.scale_log2;
  const size_t page_bytes = (size_t)ps * a.hkv * C::ROWB;
  const size_t head_off = (size_t)h_kv * C::ROWB;
  const size_t slot_stride = (size_t)a.hkv * C::ROWB;

  // this wave's share of the copies of stage n into ring slot `slot`
  auto issue = [&](int n, int slot) {
    const int k0 = kbeg + n * C::SK;
    char* base = ring + slot * C::SLOT;
    const char* src[C::PWD];
    uint32_t dst[C::PWD];
#pragma unroll
    for (int u = 0; u < C::PWD; ++u) {
      const int t = wave * C::PWD + u;           // copy index within the stage
      const bool isv = t >= C::TILE_DMA;
      const int tj = isv ? t - C::TILE_DMA : t;  // 1 KiB block within the tile
      const int p = tj * 64 + lane;
      const int r = p / C::CPR;
      const int pos = p % C::CPR;
      int key = k0 + r;
      key = key < kend ? key : kend - 1;
      const int pg = ptab[(key >> ps_shift) - pfirst];
      const size_t off = (size_t)pg * page_bytes + (size_t)(key & (ps - 1)) * slot_stride + head_off;
      src[u] = (isv ? vpool : kpool) + off + 16 * (pos ^ (isv ? C::fv(r) : C::fk(r)));
      dst[u] = lds_addr(base + (isv ? C::TILE : 0) + tj * 1024);
    }
#pragma unroll
    for (int u = 0; u < C::PWD; ++u) dma16(src[u], dst[u]);
  };

  // Stages are issued AHEAD stages before they are computed, before waiting
  // for the stage at hand.  A one-wave workgroup has finished stage n-1 when
  // it issues stage n+AHEAD into that stage's slot; with several waves the
  // slot of stage n-2 is reused instead, which every wave left behind before
  // the previous barrier.
  constexpr int AHEAD = NW == 1 ? C::NS - 1 : C::NS - 2;
  static_assert(AHEAD >= 1, "ring too shallow");
#pragma unroll
  for (int p = 0; p < AHEAD; ++p)
    if (p < nst) issue(p, p);

  int slot = 0;
  for (int n = 0; n < nst; ++n) {
    if (n + AHEAD < nst) {
      int nslot = slot + AHEAD;
      nslot = nslot >= C::NS ? nslot - C::NS : nslot;
      issue(n + AHEAD, nslot);
    }
    // own copies of stage n done (later stages may still be in flight) ...
    const int later = nst - 1 - n;
    wait_stages<C::PWD, AHEAD>(later < AHEAD ? later : AHEAD);
    // ... and everyone's
    if constexpr (NW > 1) __syncthreads();
    const char* kt = ring + slot * C::SLOT;
    const char* vt = kt + C::TILE;
    const int k0 = kbeg + n * C::SK;
    const bool needmask = k0 + C::SK > kend;

    if constexpr (SK == 16) {
      // ---- 16-key stage: S^T row rho = stage key rho; lane (q16, g) gets keys 4g .. 4g+3
      f32x4_t sc[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) sc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const char* krow = kt + q16 * C::ROWB;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((4 * s + g) ^ C::fk(q16)));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          sc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][s], sc[qb], 0, 0, 0);
      }
      s16x4_t pt[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mr = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = sc[qb][e];
          if (needmask && k0 + 4 * g + e >= kend) x = -__builtin_inff();
          sc[qb][e] = x;
          mr = fmaxf(mr, x);
        }
        mr = fmaxf(mr, __shfl_xor(mr, 16));
        mr = fmaxf(mr, __shfl_xor(mr, 32));
        const float mx = mr * c;
        const bool grow = mx > m[qb] + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float mn = grow ? mx : m[qb];
          const float al = fast_exp2(m[qb] - mn);
          l[qb] *= al;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= al;
          m[qb] = mn;
        }
        float p4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p4[e] = fast_exp2(__builtin_fmaf(sc[qb][e], c, -m[qb]));
        l[qb] += (p4[0] + p4[1]) + (p4[2] + p4[3]);
        const u32x2_t pk = {pack_bf16x2(p4[0], p4[1]), pack_bf16x2(p4[2], p4[3])};
        pt[qb] = __builtin_bit_cast(s16x4_t, pk);
      }
      // ---- O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: V^T lane (d, g) = keys 4g .. 4g+3
      const int sp = q16 >> 2;
      const int av = q16 & 3;
      const int vr = 4 * g + sp;
#pragma unroll
      for (int dbl = 0; dbl < NDB; ++dbl) {
        const int db = ds * NDB + dbl;
        const int chunk = 2 * db + (av >> 1);
        const s16x4_t vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            PS_LDS_PTR(s16x4_t, vt + vr * C::ROWB + 16 * (chunk ^ C::fv(vr)) + 8 * (av & 1)));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[qb][dbl] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pt[qb], o[qb][dbl], 0, 0, 0);
      }
    } else {
      // ---- 32-key stage: block j, S^T row rho (= q16) is stage key 8 (rho/4) + 4 j + rho%4,
      // so that lane (q16, g) holds the 8 consecutive keys 8g .. 8g+7
      f32x4_t sc[2][NQB];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sc[j][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int kr = 8 * (q16 >> 2) + 4 * j + (q16 & 3);
        const char* krow = kt + kr * C::ROWB;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          bf16x8_t kf;
          if constexpr (KDT == DT_BF16) {
            kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ((4 * s + g) ^ C::fk(kr)));
          } else {
            const u32x2_t w = *reinterpret_cast<const u32x2_t*>(
                krow + 16 * ((2 * s + (g >> 1)) ^ C::fk(kr)) + 8 * (g & 1));
            kf = fp8x8_to_bf16x8(w[0], w[1]);
          }
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            sc[j][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][s], sc[j][qb], 0, 0, 0);
        }
      }
      bf16x8_t pt[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mr = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = sc[j][qb][e];
            if (needmask && k0 + 8 * g + 4 * j + e >= kend) x = -__builtin_inff();
            sc[j][qb][e] = x;
            mr = fmaxf(mr, x);
          }
        mr = fmaxf(mr, __shfl_xor(mr, 16));
        mr = fmaxf(mr, __shfl_xor(mr, 32));
        const float mx = mr * c;
        const bool grow = mx > m[qb] + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float mn = grow ? mx : m[qb];
          const float al = fast_exp2(m[qb] - mn);
          l[qb] *= al;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= al;
          m[qb] = mn;
        }
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = fast_exp2(__builtin_fmaf(sc[j][qb][e], c, -m[qb]));
            pt[qb][4 * j + e] = (__bf16)p;
            psum += p;
          }
        l[qb] += psum;
      }
      // ---- O^T += V^T P^T over the 32 keys of the stage, this wave's columns
#pragma unroll
      for (int dbl = 0; dbl < NDB; ++dbl) {
        const int db = ds * NDB + dbl;
        bf16x8_t vf;
        if constexpr (KDT == DT_BF16) {
          const int sp = q16 >> 2;
          const int av = q16 & 3;
          const int chunk = 2 * db + (av >> 1);
          const int r1 = 8 * g + sp;
          const int r2 = r1 + 4;
          const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              PS_LDS_PTR(s16x4_t, vt + r1 * C::ROWB + 16 * (chunk ^ C::fv(r1)) + 8 * (av & 1)));
          const s16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              PS_LDS_PTR(s16x4_t, vt + r2 * C::ROWB + 16 * (chunk ^ C::fv(r2)) + 8 * (av & 1)));
          const s16x8_t v = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
          vf = __builtin_bit_cast(bf16x8_t, v);
        } else {
          const int sp = q16 >> 1;
          const int av = q16 & 1;
          const int r1 = 8 * g + sp;
          const i32x2_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              PS_LDS_PTR(i32x2_t, vt + r1 * C::ROWB + 16 * (db ^ C::fv(r1)) + 8 * av));
          vf = fp8x8_to_bf16x8((uint32_t)w[0], (uint32_t)w[1]);
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[qb][dbl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt[qb], o[qb][dbl], 0, 0, 0);
      }
    }
    slot = slot + 1 == C::NS ? 0 : slot + 1;
  }

  // ---- partial result of this split for the wave's rows and columns:
  // O_s = acc / l, LSE_s = m + log2 l (l summed over the row's four lanes)
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float lt = l[qb] + __shfl_xor(l[qb], 16);
    lt += __shfl_xor(lt, 32);
    const int r = (rg * NQB + qb) * 16 + q16;
    if (r >= a.rows) continue;
    const bool empty = !(lt > 0.f);
    const float inv = empty ? 0.f : 1.0f / lt;
    const size_t prow = (((size_t)b * a.hkv + h_kv) * a.n_splits + it.split) * a.rows + r;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int dbl = 0; dbl < NDB; ++dbl) {
      const f32x4_t v = o[qb][dbl] * inv;
      *reinterpret_cast<f32x4_t*>(po + 16 * (ds * NDB + dbl) + 4 * g) = v;
    }
    if (ds == 0 && g == 0) a.part_lse[prow] = empty ? -__builtin_inff() : m[qb] + fast_log2(lt);
  }
}

template <int D, int KDT, int SK, int NW, int NS, int RG, int DS, int NQB, int MAXP>
static int launch_t(const PagedArgs& a, int64_t n_blocks, hipStream_t s) {
  hipLaunchKernelGGL((paged_stream_kernel<D, KDT, SK, NW, NS, RG, DS, NQB, MAXP>), dim3((unsigned)n_blocks),
                     dim3(NW * 64), 0, s, a);
  return (int)hipGetLastError();
}

// Configurations (must agree with paged_geom in plan.h):
//  * single wave, 16-key bf16 stages, 3-slot ring, all rows (<= 16) and columns;
//  * four waves, 32-key stages, ring as deep as 128 KiB allows (<= 8).
template <int D, int KDT>
static int launch_d(const PagedArgs& a, const PagedGeom& geo, int64_t n_blocks, hipStream_t s) {
  constexpr int SLOT32 = 2 * 32 * D * Elem<KDT>::size;
  constexpr int NS4 = (131072 / SLOT32) > 8 ? 8 : (131072 / SLOT32);
  if (geo.waves == 1) {
    if constexpr (KDT == DT_BF16) {
      if (geo.stage_keys == 16 && geo.ring == 3 && geo.qblocks == 1)
        return launch_t<D, KDT, 16, 1, 3, 1, 1, 1, kStreamMaxPagesSmall>(a, n_blocks, s);
    }
    return (int)hipErrorInvalidValue;
  }
  if (geo.stage_keys != 32 || geo.ring != NS4) return (int)hipErrorInvalidValue;
  if (geo.qblocks == 1 && geo.row_groups == 1) return launch_t<D, KDT, 32, 4, NS4, 1, 4, 1, kStreamMaxPages>(a, n_blocks, s);
  if (geo.qblocks == 1 && geo.row_groups == 2) return launch_t<D, KDT, 32, 4, NS4, 2, 2, 1, kStreamMaxPages>(a, n_blocks, s);
  if (geo.qblocks == 1 && geo.row_groups == 4) return launch_t<D, KDT, 32, 4, NS4, 4, 1, 1, kStreamMaxPages>(a, n_blocks, s);
  if (geo.qblocks == 2 && geo.row_groups == 2) return launch_t<D, KDT, 32, 4, NS4, 2, 2, 2, kStreamMaxPages>(a, n_blocks, s);
  return (int)hipErrorInvalidValue;
}

int launch_paged_stream(const PagedArgs& a, int d, int kv_dtype, const PagedGeom& geo, int64_t n_blocks,
                        void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kv_dtype == DT_BF16) {
    switch (d) {
      case 64: return launch_d<64, DT_BF16>(a, geo, n_blocks, s);
      case 128: return launch_d<128, DT_BF16>(a, geo, n_blocks, s);
      case 256: return launch_d<256, DT_BF16>(a, geo, n_blocks, s);
    }
  } else if (kv_dtype == DT_FP8) {
    switch (d) {
      case 64: return launch_d<64, DT_FP8>(a, geo, n_blocks, s);
      case 128: return launch_d<128, DT_FP8>(a, geo, n_blocks, s);
      case 256: return launch_d<256, DT_FP8>(a, geo, n_blocks, s);
    }
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace psattn
