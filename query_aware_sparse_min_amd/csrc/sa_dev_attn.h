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
};

// Attend to pages lst[j0 .. j1) (lst == nullptr: logical pages j0 .. j1) of
// list (b, h) and write the workgroup's partial records to part[G][kPartStride].
// rlst (optional; LDS or memory written before the launch) holds the pages
// already resolved to (physical page << 4) | (valid tokens - 1), read with
// plain loads; the page table is then not read.
// PW: pages each wave loads per iteration (PW * 8 row loads in flight per lane).
// COH: lst is read and the partials are written device-coherently; ENC: the
// partial words are stored as (bits ^ kPartSentinel).
template <int KT, int QT, int G, int PW = 2, bool COH = false, int NW = 4, bool ENC = false>
__device__ __forceinline__ void attend_range(const void* __restrict__ q, const void* __restrict__ k,
                             const void* __restrict__ v, const uint16_t* __restrict__ ks,
                             const uint16_t* __restrict__ vs, int num_pages, int hkv, int b, int h,
                             const int32_t* __restrict__ pt_row, int L, const int32_t* lst, int j0,
                             int j1, float scale_log2, float* __restrict__ part,
                             AttnSmem<G, NW>& sm, const int32_t* rlst = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int hq = hkv * G;
  const int np = (L + kPage - 1) / kPage;

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

  // Resolve this wave's pages j = j0 + wave + NW * x (x < 64) up front: lane x
  // loads list entry x, then its page-table entry, so the list and the page
  // table cost one memory round trip each instead of one per page.
  int my_pp = -1, my_nv = 0;
  if (rlst) {
    const int j = j0 + wave + NW * lane;
    const int32_t r = j < j1 ? rlst[j] : -1;
    if (r >= 0) {
      my_pp = r >> 4;
      my_nv = (r & 15) + 1;
    }
  } else {
    const int j = j0 + wave + NW * lane;
    int p = -1;
    if (j < j1) p = lst ? ld_x<COH>(lst + j) : j;
    if (p >= 0 && p < np) {
      const int pp = pt_row[p];
      if (pp >= 0 && pp < num_pages) {
        my_pp = pp;
        my_nv = min(kPage, L - p * kPage);
      }
    }
  }
  auto page_of = [&](int j) -> PageRef {
    PageRef pr{-1, 0};
    if (j >= j1) return pr;
    const int x = (j - j0 - wave) / NW;  // wave-uniform
    if (x < 64) {
      pr.pp = __builtin_amdgcn_readlane(my_pp, x);
      pr.nv = __builtin_amdgcn_readlane(my_nv, x);
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
    const int p = lst ? ld_x<COH>(lst + j) : j;
    if (p < 0 || p >= np) return pr;
    const int pp = pt_row[p];
    if (pp < 0 || pp >= num_pages) return pr;
    pr.pp = pp;
    pr.nv = min(kPage, L - p * kPage);
    return pr;
  };

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
      const bool live = pg[u].pp >= 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
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
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += blockDim.x) {
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
    auto put = [&](int i, float x) {
      if constexpr (ENC) st_x<COH>(reinterpret_cast<uint32_t*>(part) + i, __float_as_uint(x) ^ kPartSentinel);
      else st_x<COH>(part + i, x);
    };
    put(g * kPartStride + dim, a);
    if (dim == 0) {
      put(g * kPartStride + kHeadDim, M);
      put(g * kPartStride + kHeadDim + 1, ls);
    }
  }
}

// Merge ns partial records part[ns][G][kPartStride] of one list into
// out[G][128]: out = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  The
// workgroup's threads form P = blockDim / (G * 128) groups (at least one);
// group p folds splits p, p + P, p + 2P, ... into a running (M, acc, sum),
// fetching C splits per memory round trip, and the groups are combined
// through lds (3 * blockDim floats).  The order is fixed, so the result is
// deterministic.  COH: partials are read device-coherently.  ENC: partials are
// stored as (bits ^ kPartSentinel) by other workgroups, 0 while not yet
// written; such words are re-read until they arrive (bounded; on timeout
// *err |= 4).  All threads call.
template <bool COH = false, bool ENC = false, int C = 16>
__device__ __forceinline__ void merge_list(const float* __restrict__ part, int ns, int G,
                                           float* __restrict__ out, float* __restrict__ lds,
                                           uint32_t* err = nullptr) {
  const int no = G * kHeadDim;
  const int nt = blockDim.x;
  const int P = nt / no > 1 ? nt / no : 1;
  // folds splits first, first + step, ... (< ns) of output o into (M, a, lsum)
  auto fold = [&](int o, int first, int step, float& M, float& a, float& lsum) {
    const int g = o / kHeadDim, dim = o % kHeadDim;
    for (int s0 = first; s0 < ns; s0 += C * step) {
      float av[C], mv[C], lv[C];
      if constexpr (ENC) {
        const uint32_t* pw = reinterpret_cast<const uint32_t*>(part);
        uint32_t aw[C], mw[C], lw[C];
        auto rec = [&](int j) { return ((size_t)min(s0 + j * step, ns - 1) * G + g) * kPartStride; };
#pragma unroll
        for (int j = 0; j < C; ++j) {  // unconditional loads (clamped split) stay in flight together
          aw[j] = ld_x<true>(pw + rec(j) + dim);
          mw[j] = ld_x<true>(pw + rec(j) + kHeadDim);
          lw[j] = ld_x<true>(pw + rec(j) + kHeadDim + 1);
        }
        bool missing = false;
#pragma unroll
        for (int j = 0; j < C; ++j) missing |= (aw[j] == 0u) | (mw[j] == 0u) | (lw[j] == 0u);
        for (uint32_t spins = 0; missing; ++spins) {  // records not yet landed: re-read those words
          if (spins > kPollLimit) {
            if (err) __hip_atomic_fetch_or(err, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          missing = false;
#pragma unroll
          for (int j = 0; j < C; ++j) {
            if (aw[j] == 0u) aw[j] = ld_x<true>(pw + rec(j) + dim);
            if (mw[j] == 0u) mw[j] = ld_x<true>(pw + rec(j) + kHeadDim);
            if (lw[j] == 0u) lw[j] = ld_x<true>(pw + rec(j) + kHeadDim + 1);
            missing |= (aw[j] == 0u) | (mw[j] == 0u) | (lw[j] == 0u);
          }
        }
#pragma unroll
        for (int j = 0; j < C; ++j) {
          av[j] = __uint_as_float(aw[j] ^ kPartSentinel);
          mv[j] = __uint_as_float(mw[j] ^ kPartSentinel);
          lv[j] = __uint_as_float(lw[j] ^ kPartSentinel);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C; ++j) {  // unconditional loads (clamped split) stay in flight together
          const float* rec = part + ((size_t)min(s0 + j * step, ns - 1) * G + g) * kPartStride;
          av[j] = ld_x<COH>(rec + dim);
          mv[j] = ld_x<COH>(rec + kHeadDim);
          lv[j] = ld_x<COH>(rec + kHeadDim + 1);
        }
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
