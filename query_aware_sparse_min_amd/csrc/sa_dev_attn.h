// sa_dev_attn.h - flash-decoding attention of one (batch, kv-head) list over
// a range of its selected pages, inside one workgroup of NW waves, and the
// merge of the per-split partials (device code shared by the standalone
// attention kernel and the fused decode-step kernel).
//
// "Quest 完全拆解": approximate attention loads only the top-K pages through the
// page table.  "SALS长序列推理优化", SFAA: QK -> online softmax -> P@V -> rescale on
// int8 K/V gathered by the selection, rows split over cores then reduced.
// "Day 10·2": the softmax is renormalised over the selected set only.
//
// Layout of the work: the NW waves take the pages of the range in turn,
// PW at a time so that 8 * PW row loads per lane are in flight.  Lane l owns token
// row (l / 16) of a 4-row group and dimensions 8*(l % 16)..+7, so one 64-lane
// load reads four whole rows of a page.  Scores are kept in base 2
// (z = q.k * scale * log2 e); each wave keeps (max, sum, acc) per query head;
// the workgroup folds its waves through LDS into one partial record
// {acc[128], max, sum} per query head.
#pragma once

#include <type_traits>

#include "sa_internal.h"

namespace sa {

constexpr int kPartStride = kHeadDim + 2;  // acc[d], max (base 2), sum

template <int G, int NW = 4>
struct AttnSmem {
  float acc[NW][G][kHeadDim];
  float m[NW][G], l[NW][G];
};

// 8 elements of a K/V row as raw words (widened when used).
template <int DT>
struct Raw8;
template <>
struct Raw8<SA_BF16> {
  uint4 w;
  __device__ __forceinline__ void load(const void* base, size_t e) {
    w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
};
template <>
struct Raw8<SA_F32> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, size_t e) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};
template <>
struct Raw8<SA_I8> {
  uint2 w;
  __device__ __forceinline__ void load(const void* base, size_t e) {
    w = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(base) + e);
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (float)(int8_t)(w.x >> (8 * i));
      x[4 + i] = (float)(int8_t)(w.y >> (8 * i));
    }
  }
};

struct PageRef {
  int pp;  // physical page, -1 if the slot is empty
  int nv;  // valid tokens
  uint32_t mask = 0xFFFFFFFFu;  // query heads of the group that attend to the page
};

// The pages j = j0 + wave, j0 + wave + NW, ... (< j1) that one wave takes from
// a list: lst[j] (lst == nullptr: logical page j) through the page table, or
// rlst[j] already resolved to (physical page << 4) | (valid tokens - 1).  The
// first 64 are resolved up front, lane x holding the x-th, so the list and the
// page table cost one memory round trip each instead of one per page.
template <bool COH, int NW>
struct WavePages {
  const int32_t* pt_row;
  const int32_t* lst;
  const int32_t* rlst;
  int j0, j1, np, num_pages, L, wave;
  bool masked;
  int my_pp = -1, my_nv = 0;
  uint32_t my_mask = 0xFFFFFFFFu;

  // jcap >= j1 bounds the list entries that may be read before j1 is known
  // (-1: j1), so that the list read need not wait for the list length.
  // masked: list entries are (head mask << 16) | logical page.
  __device__ __forceinline__ WavePages(const int32_t* pt_row_, const int32_t* lst_,
                                       const int32_t* rlst_, int j0_, int j1_, int L_,
                                       int num_pages_, int jcap = -1, bool masked_ = false)
      : pt_row(pt_row_), lst(lst_), rlst(rlst_), j0(j0_), j1(j1_),
        np((L_ + kPage - 1) / kPage), num_pages(num_pages_), L(L_),
        wave((int)(threadIdx.x >> 6)), masked(masked_) {
    const int lane = threadIdx.x & 63;
    const int j = j0 + wave + NW * lane;
    if (rlst) {
      const int32_t r = j < j1 ? rlst[j] : -1;
      if (r >= 0) {
        my_pp = r >> 4;
        my_nv = (r & 15) + 1;
      }
    } else {
      int p = -1;
      if (j < (jcap < 0 ? j1 : jcap)) p = lst ? ld_x<COH>(lst + j) : j;
      if (j >= j1) p = -1;
      if (masked && p != -1) {
        my_mask = (uint32_t)p >> 16;
        p &= 0xFFFF;
      }
      if (p >= 0 && p < np) {
        const int pp = pt_row[p];
        if (pp >= 0 && pp < num_pages) {
          my_pp = pp;
          my_nv = min(kPage, L - p * kPage);
        }
      }
    }
  }
  // the page of wave-uniform j
  __device__ __forceinline__ PageRef operator()(int j) const {
    PageRef pr{-1, 0};
    if (j >= j1) return pr;
    const int x = (j - j0 - wave) / NW;  // wave-uniform
    if (x < 64) {
      pr.pp = __builtin_amdgcn_readlane(my_pp, x);
      pr.nv = __builtin_amdgcn_readlane(my_nv, x);
      if (masked) pr.mask = (uint32_t)__builtin_amdgcn_readlane((int)my_mask, x);
      return pr;
    }
    if (rlst) {  // wave with more than 64 pages
      const int32_t r = rlst[j];
      if (r >= 0) {
        pr.pp = r >> 4;
        pr.nv = (r & 15) + 1;
      }
      return pr;
    }
    int p = lst ? ld_x<COH>(lst + j) : j;
    if (masked) {
      pr.mask = (uint32_t)p >> 16;
      p &= 0xFFFF;
    }
    if (p < 0 || p >= np) return pr;
    const int pp = pt_row[p];
    if (pp < 0 || pp >= num_pages) return pr;
    pr.pp = pp;
    pr.nv = min(kPage, L - p * kPage);
    return pr;
  }
};

// Folds the NW waves' (max, sum, acc) of every query head, which every wave
// has stored to sm.m / sm.l / sm.acc, into the workgroup's partial records
// part[G][kPartStride].  COH: stored device-coherently.  All threads call.
// W0: wave 0 alone stores the records, and every wave's earlier stores have
// completed at the barrier, so wave 0 can publish the records (wait for its
// own stores, then signal) without another barrier.
template <int G, int NW, bool COH, bool W0 = false>
__device__ __forceinline__ void put_partials(AttnSmem<G, NW>& sm, float* __restrict__ part) {
  if constexpr (W0) stores_done();
  __syncthreads();
  if (W0 && threadIdx.x >= 64) return;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += (W0 ? 64 : (int)blockDim.x)) {
    const int g = idx / kHeadDim, dim = idx % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][g]);
    float a = 0.0f, ls = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(sm.m[w][g] - M);
        a = fmaf(sm.acc[w][g][dim], f, a);
        ls = fmaf(sm.l[w][g], f, ls);
      }
    }
    auto put = [&](int i, float x) { st_x<COH>(part + i, x); };
    put(g * kPartStride + dim, a);
    if (dim == 0) {
      put(g * kPartStride + kHeadDim, M);
      put(g * kPartStride + kHeadDim + 1, ls);
    }
  }
}

// Attend to pages lst[j0 .. j1) (lst == nullptr: logical pages j0 .. j1) of
// list (b, h) and write the workgroup's partial records to part[G][kPartStride].
// rlst (optional; LDS or memory written before the launch) holds the pages
// already resolved to (physical page << 4) | (valid tokens - 1), read with
// plain loads; the page table is then not read.
// PW: pages each wave loads per iteration (PW * 8 row loads in flight per lane).
// COH: lst is read and the partials are written device-coherently.
template <int KT, int QT, int G, int PW = 2, bool COH = false, int NW = 4, bool W0 = false>
__device__ __forceinline__ void attend_range(const void* __restrict__ q, const void* __restrict__ k,
                             const void* __restrict__ v, const uint16_t* __restrict__ ks,
                             const uint16_t* __restrict__ vs, int num_pages, int hkv, int b, int h,
                             const int32_t* __restrict__ pt_row, int L, const int32_t* lst, int j0,
                             int j1, float scale_log2, float* __restrict__ part,
                             AttnSmem<G, NW>& sm, const int32_t* rlst = nullptr,
                             int jcap = -1, bool masked = false) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int hq = hkv * G;

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) load8<QT>(q, ((size_t)b * hq + (size_t)h * G + g) * kHeadDim + 8 * c, qv[g]);

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
  }

  const WavePages<COH, NW> page_of(pt_row, lst, rlst, j0, j1, L, num_pages, jcap, masked);

  for (int jb = j0 + wave; jb < j1; jb += NW * PW) {
    PageRef pg[PW];
    Raw8<KT> kr[PW][4], vr[PW][4];
    float ksc[PW][4], vsc[PW][4];
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      pg[u] = page_of(jb + NW * u);
      const int ppl = pg[u].pp >= 0 ? pg[u].pp : 0;  // empty slot: load page 0, result unused
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const size_t tok = ((size_t)ppl * kPage + 4 * it + r) * hkv + h;
        kr[u][it].load(k, tok * kHeadDim + 8 * c);
        vr[u][it].load(v, tok * kHeadDim + 8 * c);
        if constexpr (KT == SA_I8) {
          ksc[u][it] = f16_to_f32(ks[tok]);
          vsc[u][it] = f16_to_f32(vs[tok]);
        } else {
          ksc[u][it] = vsc[u][it] = 1.0f;
        }
      }
    }
    // every K/V load of the iteration is issued before any of them is used
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      // an empty slot is masked (selects, no branch, so the loads above stay
      // where they are): all its scores are -inf and it changes nothing
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const bool live = pg[u].pp >= 0 && ((pg[u].mask >> g) & 1u);
        float z[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          float kx[8];
          kr[u][it].get(kx);
          float s = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) s = fmaf(qv[g][e], kx[e], s);
          s = sum16(s);
          z[it] = (live && 4 * it + r < pg[u].nv) ? s * (scale_log2 * ksc[u][it]) : -INFINITY;
        }
        float pm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        pm = pair32_max(pair16_max(pm));
        const float mn = fmaxf(m[g], pm);  // -inf only while nothing has been attended
        const bool none = mn == -INFINITY;
        const float alpha = none ? 1.0f : exp2f(m[g] - mn);
        float pr[4], psum = 0.0f;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          pr[it] = none ? 0.0f : exp2f(z[it] - mn);
          psum += pr[it];
          pr[it] *= vsc[u][it];
        }
        l[g] = l[g] * alpha + psum;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          float vx[8];
          vr[u][it].get(vx);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pr[it], vx[e], acc[g][e]);
        }
        m[g] = mn;
      }
    }
  }

  // fold the four token rows of each wave, then the NW waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = pair32_sum(pair16_sum(l[g]));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = pair32_sum(pair16_sum(acc[g][e]));
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.acc[wave][g][8 * c + e] = acc[g][e];
      if (c == 0) {
        sm.m[wave][g] = m[g];
        sm.l[wave][g] = l[g];
      }
    }
  }
  put_partials<G, NW, COH, W0>(sm, part);
}

// ---------------------------------------------------------------- MFMA variant
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Eight consecutive K elements of a row as one bf16 MFMA operand (int8 codes
// are widened exactly: every code has at most 8 significant bits).
template <int DT>
struct KOp8;
template <>
struct KOp8<SA_BF16> {
  uint4 w;
  __device__ __forceinline__ void load(const void* base, size_t e) {
    w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
  }
  __device__ __forceinline__ bf16x8_t get() const { return __builtin_bit_cast(bf16x8_t, w); }
};
template <>
struct KOp8<SA_I8> {
  uint2 w;
  __device__ __forceinline__ void load(const void* base, size_t e) {
    w = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(base) + e);
  }
  __device__ __forceinline__ bf16x8_t get() const {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = i < 2 ? w.x : w.y;
      const int sh = 16 * (i & 1);
      const float lo = (float)(int8_t)(word >> sh), hi = (float)(int8_t)(word >> (sh + 8));
      o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  }
};

// The 32 consecutive K elements of a lane's row slice (four MFMA operands of
// eight): bf16 as four 16-byte loads, int8 codes as two.
template <int DT>
struct KOp32;
template <>
struct KOp32<SA_BF16> {
  KOp8<SA_BF16> o[4];
  __device__ __forceinline__ void load(const void* base, size_t e) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) o[kk].load(base, e + 8 * kk);
  }
  __device__ __forceinline__ bf16x8_t get(int kk) const { return o[kk].get(); }
};
template <>
struct KOp32<SA_I8> {
  uint4 w[2];
  __device__ __forceinline__ void load(const void* base, size_t e) {
    const int8_t* p = static_cast<const int8_t*>(base) + e;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) w[hh] = *reinterpret_cast<const uint4*>(p + 16 * hh);
  }
  __device__ __forceinline__ bf16x8_t get(int kk) const {
    KOp8<SA_I8> o;
    o.w = (kk & 1) ? make_uint2(w[kk >> 1].z, w[kk >> 1].w) : make_uint2(w[kk >> 1].x, w[kk >> 1].y);
    return o.get();
  }
};

// Value of lane g of each 16-lane row (DPP row_newbcast).
template <int g>
__device__ __forceinline__ float row_bcast(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v),
                                                               0x150 + g, 0xF, 0xF, false));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// attend_range for G (<= 16) bf16 query heads per kv-head, with the scores
// Q K^T of a page on the matrix cores: four v_mfma_f32_16x16x32_bf16 per page
// compute the 16 tokens x 16 head-slots score tile (heads >= G are zero).
// The A operand is the page's K: lane l supplies row l % 16 as token
// 4 * (l % 4) + (l % 16) / 4 and 32 of its dimensions, (l / 16) * 32 .. + 31,
// eight per MFMA; the B operand is Q^T laid out the same way.  With that token
// order lane l ends up holding, for head l % 16, the scores of tokens
// 4 i + l / 16 (i = 0..3): exactly the tokens whose V rows it holds in the
// P V layout of attend_range (token row l / 16 of each group of four), so each
// head's weights reach the P V lanes by one row broadcast from lane g of the
// row, and P V stays on the vector ALUs in fp32 (no bf16 rounding of weights).
// int8 K / V: the codes enter the MFMA exactly; the per-token scales multiply
// the scores and the weights.  Partials as attend_range.
// PW: pages each wave loads per iteration, all in flight before any is used.
// rlst / COH: as attend_range (pages already resolved to (physical page << 4) |
// (valid tokens - 1), read from LDS; partial records stored device-coherently).
template <int KT, int G, int NW = 4, int PW = 1, bool COH = false>
__device__ __forceinline__ void attend_range_mfma(const void* __restrict__ q,
                                                  const void* __restrict__ k,
                                                  const void* __restrict__ v,
                                                  const uint16_t* __restrict__ ks,
                                                  const uint16_t* __restrict__ vs, int num_pages,
                                                  int hkv, int b, int h,
                                                  const int32_t* __restrict__ pt_row, int L,
                                                  const int32_t* lst, int j0, int j1,
                                                  float scale_log2, float* __restrict__ part,
                                                  AttnSmem<G, NW>& sm, int jcap = -1,
                                                  bool masked = false,
                                                  const int32_t* rlst = nullptr) {
  static_assert(G >= 1 && G <= 16, "one MFMA column per query head");
  static_assert(KT == SA_BF16 || KT == SA_I8, "K enters the MFMA as bf16");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, qg = lane >> 4;  // MFMA column (head) and row group
  const int r = qg, c = n;                  // P V layout: token row in a group of 4, dims 8c..
  const int hq = hkv * G;
  const int tok_a = 4 * (n & 3) + (n >> 2);  // the token of this lane's A row

  bf16x8_t qb[4];
  {
    uint4 w[4] = {};
    if (n < G) {
      const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) +
                                                       ((size_t)b * hq + (size_t)h * G + n) * kHeadDim +
                                                       32 * qg);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) w[kk] = qp[kk];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = __builtin_bit_cast(bf16x8_t, w[kk]);
  }

  float mrun = -INFINITY, lpart = 0.0f;  // head n: running max; this lane's tokens' weight sum
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;

  const WavePages<false, NW> page_of(pt_row, lst, rlst, j0, j1, L, num_pages, jcap, masked);
  for (int jb = j0 + wave; jb < j1; jb += NW * PW) {
    PageRef pg[PW];
    KOp32<KT> kr[PW];
    Raw8<KT> vr[PW][4];
    // int8: the K and V scales (fp16 bits) of token lane % 16 of the page; a
    // lane takes those of its own tokens from the lanes that hold them
    uint32_t kscw[PW], vscw[PW];
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      pg[u] = page_of(jb + NW * u);
      const size_t ppl = pg[u].pp >= 0 ? (size_t)pg[u].pp : 0;  // empty slot: load page 0, result unused
      const size_t row = (ppl * kPage + tok_a) * hkv + h;
      kr[u].load(k, row * kHeadDim + 32 * qg);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const size_t tv = (ppl * kPage + 4 * it + r) * hkv + h;
        vr[u][it].load(v, tv * kHeadDim + 8 * c);
      }
      if constexpr (KT == SA_I8) {
        const size_t ts = (ppl * kPage + (lane & 15)) * hkv + h;
        kscw[u] = ks[ts];
        vscw[u] = vs[ts];
      }
    }
    // every load of the iteration is issued before any of them is used
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      float ksc[4], vsc[4];  // tokens 4 i + qg
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KT == SA_I8) {
          ksc[i] = f16_to_f32((uint16_t)__builtin_amdgcn_ds_bpermute(4 * (4 * i + qg), (int)kscw[u]));
          vsc[i] = f16_to_f32((uint16_t)__builtin_amdgcn_ds_bpermute(4 * (4 * i + qg), (int)vscw[u]));
        } else {
          ksc[i] = vsc[i] = 1.0f;
        }
      }
      f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[u].get(kk), qb[kk], z, 0, 0, 0);

      const bool live = pg[u].pp >= 0 && n < G && ((pg[u].mask >> n) & 1u);
      float zz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)  // token 4 i + qg
        zz[i] = (live && 4 * i + qg < pg[u].nv) ? z[i] * (scale_log2 * ksc[i]) : -INFINITY;
      float pm = fmaxf(fmaxf(zz[0], zz[1]), fmaxf(zz[2], zz[3]));
      pm = pair32_max(pair16_max(pm));  // over the page's 16 tokens, for head n
      const float mn = fmaxf(mrun, pm);
      const bool none = mn == -INFINITY;
      const float alpha = none ? 1.0f : exp2f(mrun - mn);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = none ? 0.0f : exp2f(zz[i] - mn);
      lpart = fmaf(lpart, alpha, (p[0] + p[1]) + (p[2] + p[3]));
      mrun = mn;

      static_for<0, G>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const float ag = row_bcast<g>(alpha);
        float pw[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) pw[it] = row_bcast<g>(p[it]) * vsc[it];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          float vx[8];
          vr[u][it].get(vx);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw[it], vx[e], acc[g][e]);
        }
      });
    }
  }

  // fold the four token rows of each wave, then the NW waves
  const float lsum = pair32_sum(pair16_sum(lpart));
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = pair32_sum(pair16_sum(acc[g][e]));
  if (qg == 0 && n < G) {
    sm.m[wave][n] = mrun;
    sm.l[wave][n] = lsum;
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.acc[wave][g][8 * c + e] = acc[g][e];
  }
  put_partials<G, NW, COH>(sm, part);
}

// Merge ns partial records part[ns][G][kPartStride] of one list into
// out[G][128]: out = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), for the
// query heads g0 .. g0 + gn - 1 (gn < 0: all G).  The workgroup's threads
// form P = blockDim / (gn * 128) groups (at least one);
// group p folds splits p, p + P, p + 2P, ... into a running (M, acc, sum),
// fetching C splits per memory round trip, and the groups are combined
// through lds (3 * blockDim floats).  The order is fixed, so the result is
// deterministic.  COH: partials are read device-coherently (written by other
// workgroups of the same launch).  All threads call.
// merge_list by one wave, without LDS or barriers: lane l folds output
// dimensions l and l + 64 of each of the G query heads over the ns records
// part[ns][G][kPartStride] in order, C records per memory round trip (the same
// arithmetic as merge_list's single group).  Only the calling wave takes part.
template <int G, bool COH = false, int C = (G <= 2 ? 8 : (G <= 8 ? 4 : 1))>
__device__ __forceinline__ void merge_list_wave(const float* __restrict__ part, int ns,
                                                float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  float M[G], a0[G], a1[G], lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    M[g] = -INFINITY;
    a0[g] = a1[g] = lsum[g] = 0.0f;
  }
  for (int s0 = 0; s0 < ns; s0 += C) {
    float av0[C][G], av1[C][G], mv[C][G], lv[C][G];
#pragma unroll
    for (int j = 0; j < C; ++j) {  // unconditional loads (clamped record) stay in flight together
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float* rec = part + ((size_t)min(s0 + j, ns - 1) * G + g) * kPartStride;
        av0[j][g] = ld_x<COH>(rec + lane);
        av1[j][g] = ld_x<COH>(rec + 64 + lane);
        mv[j][g] = ld_x<COH>(rec + kHeadDim);
        lv[j][g] = ld_x<COH>(rec + kHeadDim + 1);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < C; ++j)
        if (s0 + j >= ns) lv[j][g] = 0.0f;
      float Mc = M[g];
#pragma unroll
      for (int j = 0; j < C; ++j)
        if (lv[j][g] > 0.0f) Mc = fmaxf(Mc, mv[j][g]);
      if (Mc == -INFINITY) continue;  // nothing attended so far
      const float r = exp2f(M[g] - Mc);  // 0 when M is still -inf
      a0[g] *= r;
      a1[g] *= r;
      lsum[g] *= r;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        if (lv[j][g] > 0.0f) {
          const float w = exp2f(mv[j][g] - Mc);
          a0[g] = fmaf(av0[j][g], w, a0[g]);
          a1[g] = fmaf(av1[j][g], w, a1[g]);
          lsum[g] = fmaf(lv[j][g], w, lsum[g]);
        }
      }
      M[g] = Mc;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    out[g * kHeadDim + lane] = lsum[g] > 0.0f ? a0[g] / lsum[g] : 0.0f;
    out[g * kHeadDim + 64 + lane] = lsum[g] > 0.0f ? a1[g] / lsum[g] : 0.0f;
  }
}

template <bool COH = false, int C = 16>
__device__ __forceinline__ void merge_list(const float* __restrict__ part, int ns, int G,
                                           float* __restrict__ out, float* __restrict__ lds,
                                           int g0 = 0, int gn = -1) {
  if (gn < 0) gn = G;
  out += (size_t)g0 * kHeadDim;
  const int no = gn * kHeadDim;
  const int nt = blockDim.x;
  const int P = nt / no > 1 ? nt / no : 1;
  // folds splits first, first + step, ... (< ns) of output o into (M, a, lsum)
  auto fold = [&](int o, int first, int step, float& M, float& a, float& lsum) {
    const int g = g0 + o / kHeadDim, dim = o % kHeadDim;
    for (int s0 = first; s0 < ns; s0 += C * step) {
      float av[C], mv[C], lv[C];
#pragma unroll
      for (int j = 0; j < C; ++j) {  // unconditional loads (clamped split) stay in flight together
        const float* rec = part + ((size_t)min(s0 + j * step, ns - 1) * G + g) * kPartStride;
        av[j] = ld_x<COH>(rec + dim);
        mv[j] = ld_x<COH>(rec + kHeadDim);
        lv[j] = ld_x<COH>(rec + kHeadDim + 1);
      }
#pragma unroll
      for (int j = 0; j < C; ++j)
        if (s0 + j * step >= ns) lv[j] = 0.0f;
      float Mc = M;
#pragma unroll
      for (int j = 0; j < C; ++j)
        if (lv[j] > 0.0f) Mc = fmaxf(Mc, mv[j]);
      if (Mc == -INFINITY) continue;  // nothing attended so far
      const float r = exp2f(M - Mc);  // 0 when M is still -inf
      a *= r;
      lsum *= r;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        if (lv[j] > 0.0f) {
          const float w = exp2f(mv[j] - Mc);
          a = fmaf(av[j], w, a);
          lsum = fmaf(lv[j], w, lsum);
        }
      }
      M = Mc;
    }
  };
  if (P == 1) {
    for (int o = threadIdx.x; o < no; o += nt) {
      float M = -INFINITY, a = 0.0f, lsum = 0.0f;
      fold(o, 0, 1, M, a, lsum);
      out[o] = lsum > 0.0f ? a / lsum : 0.0f;
    }
    return;
  }
  const int t = threadIdx.x;
  float M = -INFINITY, a = 0.0f, lsum = 0.0f;
  if (t < P * no) fold(t % no, t / no, P, M, a, lsum);
  lds[t] = M;
  lds[nt + t] = a;
  lds[2 * nt + t] = lsum;
  __syncthreads();
  if (t < no) {
    float Mx = -INFINITY;
    for (int p = 0; p < P; ++p)
      if (lds[2 * nt + p * no + t] > 0.0f) Mx = fmaxf(Mx, lds[p * no + t]);
    float at = 0.0f, lt = 0.0f;
    if (Mx != -INFINITY) {
      for (int p = 0; p < P; ++p) {
        const float lp = lds[2 * nt + p * no + t];
        if (lp > 0.0f) {
          const float w = exp2f(lds[p * no + t] - Mx);
          at = fmaf(lds[nt + p * no + t], w, at);
          lt = fmaf(lp, w, lt);
        }
      }
    }
    out[t] = lt > 0.0f ? at / lt : 0.0f;
  }
}

}  // namespace sa
