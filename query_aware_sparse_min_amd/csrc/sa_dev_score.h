// sa_dev_score.h - Quest page scores of a range of pages of one list inside
// one workgroup of NW waves (device code shared by the standalone scorer and
// the fused decode-step kernel).
//
// "Quest 完全拆解" explainer, upper bound from min/max metadata and the GQA
// section: score = max over the group's query heads g of
// sum_i max(q_gi m_i, q_gi M_i), evaluated as q+ . M + q- . m with
// q+ = max(q, 0), q- = min(q, 0).  Sixteen lanes own one page: lane
// (row, c) holds dimensions 16c..16c+15 of the M row (row 0) or the m row
// (row 1) of the (page, kv-head) record, as two 16-byte loads, so one pair of
// 64-lane loads covers four pages and a 16-lane all-reduce (one DPP row)
// finishes four sums at once.  With bf16 metadata and a bf16 query the
// products run as bf16 pair dot products into fp32 (q+ and q- are exact in
// bf16); otherwise as fp32 FMAs.  The metadata is head-major,
// [Hkv][num_pages][2][d], so the records of one list's pages lie next to each
// other when its pages do.
#pragma once

#include "sa_dev_attn.h"

namespace sa {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Pages [p0, p1) of list (b, h), at most 4 * NW * IT pages, p1 <= the page-table
// row length max_pages; pages at or beyond the list's page count n score -inf.
// n is ceil(min(*len_b, 16 max_pages) / 16), read after the page-table and
// metadata loads have been issued so that they need not wait for it; the
// function returns n.  sc_row: the list's scores (device-coherent stores when
// COH; KEYS: stored as order_key() words instead of floats).  pp_out
// (optional, LDS): the physical page of page p0 + j at [j], -1
// when the page is invalid or its page-table entry is out of range.  PH: each
// query head's own bound instead of the group max, head g's row at
// sc_row + g * head_stride.  All 64 * NW threads call.
template <int KT, int QT, int G, int IT, bool COH = false, int NW = 4, bool KEYS = false,
          bool PH = false>
__device__ __forceinline__ int quest_score_range(const void* __restrict__ q,
                                                  const void* __restrict__ meta, int num_pages,
                                                  int hkv, int b, int h,
                                                  const int32_t* __restrict__ pt_row, int p0,
                                                  int p1, const int32_t* __restrict__ len_b,
                                                  int max_pages, float* __restrict__ sc_row,
                                                  int32_t* pp_out = nullptr, int head_stride = 0) {
  constexpr bool kDot = KT == SA_BF16 && QT == SA_BF16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int quarter = lane >> 4, row = (lane >> 3) & 1, c = lane & 7;
  const int hq = hkv * G;

  // all loads are unconditional, from clamped in-range addresses, so that they
  // are in flight together; out-of-range results are discarded below
  int pg[IT];
  int ppg[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = p0 + 4 * (wave + NW * it) + quarter;
    pg[it] = p;
    ppg[it] = pt_row[min(p, p1 - 1)];
  }
  Raw8<KT> x[IT][2];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pp = (ppg[it] >= 0 && ppg[it] < num_pages) ? ppg[it] : 0;
    const size_t e0 = (((size_t)h * num_pages + pp) * 2 + row) * kHeadDim + 16 * c;
    x[it][0].load(meta, e0);
    x[it][1].load(meta, e0 + 8);
  }
  const int n_valid = (clamp_len(*len_b, max_pages) + kPage - 1) / kPage;
  // this lane's 16 query dimensions, q+ on M rows and q- on m rows
  float qs[kDot ? 1 : G][16];
  uint32_t qw[kDot ? G : 1][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const size_t qe = ((size_t)b * hq + (size_t)h * G + g) * kHeadDim + 16 * c;
    if constexpr (kDot) {
      Raw8<SA_BF16> r0, r1;
      r0.load(q, qe);
      r1.load(q, qe + 8);
      const uint32_t w[8] = {r0.w.x, r0.w.y, r0.w.z, r0.w.w, r1.w.x, r1.w.y, r1.w.z, r1.w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // keep the halves whose sign matches the row
        const uint32_t neg = (w[e] & 0x8000u ? 0x0000FFFFu : 0u) | (w[e] & 0x80000000u ? 0xFFFF0000u : 0u);
        qw[g][e] = w[e] & (row ? neg : ~neg);
      }
    } else {
      float t[8];
      load8<QT>(q, qe, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[g][e] = row ? fminf(t[e], 0.0f) : fmaxf(t[e], 0.0f);
      load8<QT>(q, qe + 8, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[g][8 + e] = row ? fminf(t[e], 0.0f) : fmaxf(t[e], 0.0f);
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const bool ok = pg[it] < p1 && pg[it] < n_valid && ppg[it] >= 0 && ppg[it] < num_pages;
    float best = -INFINITY;
    float per[PH ? G : 1];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.0f;
      if constexpr (kDot) {
        const uint32_t xw[8] = {x[it][0].w.x, x[it][0].w.y, x[it][0].w.z, x[it][0].w.w,
                                x[it][1].w.x, x[it][1].w.y, x[it][1].w.z, x[it][1].w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[g][e]),
                                              __builtin_bit_cast(bf16x2_t, xw[e]), s, false);
      } else {
        float xv[8];
        x[it][0].get(xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qs[g][e], xv[e], s);
        x[it][1].get(xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qs[g][8 + e], xv[e], s);
      }
      // the loaded words are used unconditionally and the page's validity is
      // applied to the sum (a select, not a branch), so no load is sunk
      s = sum16(s);
      best = fmaxf(best, s);
      if constexpr (PH) per[g] = s;
    }
    if constexpr (PH) {
      if ((lane & 15) == 0 && pg[it] < p1) {
#pragma unroll
        for (int g = 0; g < G; ++g) st_x<COH>(sc_row + (size_t)g * head_stride + pg[it], ok ? per[g] : -INFINITY);
      }
      continue;
    }
    if ((lane & 15) == 0 && pg[it] < p1) {
      const float sv = ok ? best : -INFINITY;
      if constexpr (KEYS) st_x<COH>(reinterpret_cast<uint32_t*>(sc_row) + pg[it], order_key(sv));
      else st_x<COH>(sc_row + pg[it], sv);
      if (pp_out) pp_out[pg[it] - p0] = ok ? ppg[it] : -1;
    }
  }
  return n_valid;
}

}  // namespace sa
