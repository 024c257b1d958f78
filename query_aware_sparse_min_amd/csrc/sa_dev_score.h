// sa_dev_score.h - Quest page scores of a range of pages of one list inside
// one 256-thread workgroup (device code shared by the standalone scorer and
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

// Pages [p0, p1) of list (b, h); at most 8 * IT pages.  sc_row: the list's
// scores (device-coherent stores when COH).  All 256 threads call.
template <int KT, int QT, int G, int IT, bool COH = false>
__device__ __forceinline__ void quest_score_range(const void* __restrict__ q,
                                                  const void* __restrict__ meta, int num_pages,
                                                  int hkv, int b, int h,
                                                  const int32_t* __restrict__ pt_row, int p0,
                                                  int p1, float* __restrict__ sc_row) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, row = (lane >> 4) & 1, c = lane & 15;
  const int hq = hkv * G;

  // all loads are unconditional, from clamped in-range addresses, so that they
  // are in flight together; out-of-range results are discarded below
  int pg[IT];
  int ppg[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = p0 + 2 * (wave + 4 * it) + half;
    pg[it] = p;
    ppg[it] = pt_row[min(p, p1 - 1)];
  }
  Raw8<KT> x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pp = (ppg[it] >= 0 && ppg[it] < num_pages) ? ppg[it] : 0;
    x[it].load(meta, (((size_t)h * num_pages + pp) * 2 + row) * kHeadDim + 8 * c);
  }
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
    const bool ok = pg[it] < p1 && ppg[it] >= 0 && ppg[it] < num_pages;
    float xv[8];
    if (ok) {
      x[it].get(xv);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = 0.0f;
    }
    float best = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(qs[g][e], xv[e], s);
      s = pair16_sum(sum16(s));
      best = fmaxf(best, s);
    }
    if ((lane & 31) == 0 && pg[it] < p1) st_x<COH>(sc_row + pg[it], ok ? best : -INFINITY);
  }
}

}  // namespace sa
