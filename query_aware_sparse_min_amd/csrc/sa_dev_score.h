// sa_dev_score.h - Quest page scores of a range of pages of one list inside
// one workgroup of NW waves (device code shared by the standalone scorer and
// the fused decode-step kernel).
//
// "Quest 完全拆解" explainer, upper bound from min/max metadata and the GQA
// section: score = max over the group's query heads g of
// sum_i max(q_gi m_i, q_gi M_i), evaluated as q+ . M + q- . m with
// q+ = max(q, 0), q- = min(q, 0).  A lane owns 8 dimensions of either the M
// row or the m row of a (page, kv-head) record, so one 64-lane load covers two
// pages in coalesced 256-byte rows; a 32-lane all-reduce finishes each sum.  The
// metadata is head-major, [Hkv][num_pages][2][d], so the records of one list's
// pages lie next to each other when its pages do.
#pragma once

#include "sa_dev_attn.h"

namespace sa {

// Pages [p0, p1) of list (b, h), at most 2 * NW * IT pages, p1 <= the page-table
// row length max_pages; pages at or beyond the list's page count n score -inf.
// n is ceil(min(*len_b, 16 max_pages) / 16), read after the page-table and
// metadata loads have been issued so that they need not wait for it; the
// function returns n.  sc_row: the list's scores (device-coherent stores when
// COH; KEYS: stored as order_key() words instead of floats).  pp_out
// (optional, LDS): the physical page of page p0 + j at [j], -1
// when the page is invalid or its page-table entry is out of range.  All
// 64 * NW threads call.
template <int KT, int QT, int G, int IT, bool COH = false, int NW = 4, bool KEYS = false>
__device__ __forceinline__ int quest_score_range(const void* __restrict__ q,
                                                  const void* __restrict__ meta, int num_pages,
                                                  int hkv, int b, int h,
                                                  const int32_t* __restrict__ pt_row, int p0,
                                                  int p1, const int32_t* __restrict__ len_b,
                                                  int max_pages, float* __restrict__ sc_row,
                                                  int32_t* pp_out = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, row = (lane >> 4) & 1, c = lane & 15;
  const int hq = hkv * G;

  // all loads are unconditional, from clamped in-range addresses, so that they
  // are in flight together; out-of-range results are discarded below
  int pg[IT];
  int ppg[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = p0 + 2 * (wave + NW * it) + half;
    pg[it] = p;
    ppg[it] = pt_row[min(p, p1 - 1)];
  }
  Raw8<KT> x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pp = (ppg[it] >= 0 && ppg[it] < num_pages) ? ppg[it] : 0;
    x[it].load(meta, (((size_t)h * num_pages + pp) * 2 + row) * kHeadDim + 8 * c);
  }
  const int n_valid = (clamp_len(*len_b, max_pages) + kPage - 1) / kPage;
  float qs[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float t[8];
    load8<QT>(q, ((size_t)b * hq + (size_t)h * G + g) * kHeadDim + 8 * c, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[g][e] = row ? fminf(t[e], 0.0f) : fmaxf(t[e], 0.0f);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const bool ok = pg[it] < p1 && pg[it] < n_valid && ppg[it] >= 0 && ppg[it] < num_pages;
    // unconditional use of the loaded words (a select, not a branch), so the
    // compiler cannot sink the load into a branch behind the others
    float xv[8];
    x[it].get(xv);
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = ok ? xv[e] : 0.0f;
    float best = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(qs[g][e], xv[e], s);
      s = pair16_sum(sum16(s));
      best = fmaxf(best, s);
    }
    if ((lane & 31) == 0 && pg[it] < p1) {
      const float sv = ok ? best : -INFINITY;
      if constexpr (KEYS) st_x<COH>(reinterpret_cast<uint32_t*>(sc_row) + pg[it], order_key(sv));
      else st_x<COH>(sc_row + pg[it], sv);
      if (pp_out) pp_out[pg[it] - p0] = ok ? ppg[it] : -1;
    }
  }
  return n_valid;
}

}  // namespace sa
