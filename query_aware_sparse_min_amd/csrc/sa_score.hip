// sa_score.hip - page / block scorers (step 1 of the decode step).
//
//  * Quest criticality estimation ("Quest 完全拆解" explainer, upper bound
//    from min/max metadata; GQA section): score = max over the group's query
//    heads of sum_i max(q_i m_i, q_i M_i).  The sum is evaluated in its
//    equivalent linear form q+ . M + q- . m (q+ = max(q, 0), q- = min(q, 0)):
//    a lane owns 8 dimensions of either the M row or the m row of a
//    (page, kv-head) unit, so one 64-lane load covers two units with
//    coalesced 256-byte rows, and a 32-lane tree reduction finishes each sum.
//  * SALS block scorer ("SALS长序列推理优化", QSI steps 1-3): index query =
//    group mean of q projected by P; per token s_t = scale_t * qt . c_t from
//    the int4 codes; per block a log-sum-exp of tau * s_t, kept as an online
//    (max, sum) pair in base 2 and merged across the lanes of a kv-head.
#include "sa_dev_score.h"

namespace sa {
namespace {

constexpr int kScoreIT = 2;                        // load pairs per lane
constexpr int kScorePagesPerWG = 16 * kScoreIT;     // 32 pages per workgroup

// grid (ceil(max_pages / 32), Hkv, B), block 256
template <int KT, int QT, int G>
__global__ __launch_bounds__(256) void quest_score_kernel(
    const void* __restrict__ q, const void* __restrict__ meta, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    float* __restrict__ scores) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(lens[b], max_pages);
  const int n = (L + kPage - 1) / kPage;
  const int p0 = blockIdx.x * kScorePagesPerWG;
  if (p0 >= n) return;
  quest_score_range<KT, QT, G, kScoreIT>(q, meta, num_pages, hkv, b, h, pt + (size_t)b * max_pages,
                                         p0, min(p0 + kScorePagesPerWG, n), lens + b, max_pages,
                                         scores + ((size_t)b * hkv + h) * max_pages);
}

// grid (ceil(max_units / units_per_wg), B), block 256
template <int QT>
__global__ __launch_bounds__(256) void sals_score_kernel(
    const void* __restrict__ q, int hq, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const float* __restrict__ proj, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    int unit_tokens, float tau_log2e, float* __restrict__ scores, int max_units,
    int units_per_wg) {
  __shared__ float qbar[64 * kHeadDim];  // [hkv][d] group-mean query (hkv <= 64)
  __shared__ float qt_s[64 * kRank];     // [hkv][rank] projected index query
  const int b = blockIdx.y;
  const int L = clamp_len(lens[b], max_pages);
  const int nu = (L + unit_tokens - 1) / unit_tokens;
  const int u0 = blockIdx.x * units_per_wg;
  if (u0 >= nu) return;
  const int G = hq / hkv;
  const float inv_g = 1.0f / (float)G;
  for (int i = threadIdx.x; i < hkv * kHeadDim; i += blockDim.x) {
    const int hh = i / kHeadDim, dim = i % kHeadDim;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) {
      const size_t qi = ((size_t)b * hq + (size_t)hh * G + g) * kHeadDim + dim;
      s += QT == SA_F32 ? static_cast<const float*>(q)[qi]
                        : bf16_to_f32(static_cast<const uint16_t*>(q)[qi]);
    }
    qbar[i] = s * inv_g;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < hkv * kRank; i += blockDim.x) {
    const int hh = i / kRank, j = i % kRank;
    float s = 0.0f;
    for (int dim = 0; dim < kHeadDim; ++dim) s = fmaf(qbar[hh * kHeadDim + dim], proj[dim * kRank + j], s);
    qt_s[i] = s;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tpl = 64 / hkv;  // tokens per 64-lane load
  const int tl = lane / hkv, hh = lane % hkv;
  float qt[kRank];
#pragma unroll
  for (int j = 0; j < kRank; ++j) qt[j] = qt_s[hh * kRank + j];

  const int u_end = min(u0 + units_per_wg, nu);
  for (int u = u0 + wave; u < u_end; u += 4) {
    const int t_begin = u * unit_tokens;
    const int t_end = min(t_begin + unit_tokens, L);
    float m = -INFINITY, s = 0.0f;
    for (int t0 = t_begin; t0 < t_end; t0 += tpl) {
      const int t = t0 + tl;
      if (t < t_end) {
        const int pp = pt[(size_t)b * max_pages + (t >> 4)];
        if (pp >= 0 && pp < num_pages) {
          const size_t row = ((size_t)pp * kPage + (t & 15)) * hkv + hh;
          const uint2 w = *reinterpret_cast<const uint2*>(codes + row * (kRank / 2));
          const float sc = f16_to_f32(scales[row]);
          float dot = 0.0f;
#pragma unroll
          for (int j = 0; j < kRank; ++j) {
            const uint32_t word = j < 8 ? w.x : w.y;
            const int cj = (int)(word << (28 - 4 * (j & 7))) >> 28;
            dot = fmaf(qt[j], (float)cj, dot);
          }
          const float z = tau_log2e * (sc * dot);
          if (z > m) {
            s = s * exp2f(m - z) + 1.0f;
            m = z;
          } else {
            s += exp2f(z - m);
          }
        }
      }
    }
    // merge (m, s) over the lanes that hold the same kv-head
    for (int mask = hkv; mask < 64; mask <<= 1) {
      const float m2 = __shfl_xor(m, mask, 64);
      const float s2 = __shfl_xor(s, mask, 64);
      const float mm = fmaxf(m, m2);
      s = (mm == -INFINITY) ? 0.0f : s * exp2f(m - mm) + s2 * exp2f(m2 - mm);
      m = mm;
    }
    if (tl == 0) scores[((size_t)b * hkv + hh) * max_units + u] = (m + __log2f(s)) * kLn2;
  }
}

template <int KT, int QT>
hipError_t quest_dispatch_g(int G, dim3 grid, hipStream_t st, const void* q, const void* meta,
                            const Shapes& s, const int32_t* pt, const int32_t* lens,
                            float* scores) {
#define SA_QS(GG)                                                                              \
  hipLaunchKernelGGL((quest_score_kernel<KT, QT, GG>), grid, dim3(256), 0, st, q, meta,        \
                     s.num_pages, s.Hkv, pt, lens, s.max_pages, scores)
  switch (G) {
    case 1: SA_QS(1); break;
    case 2: SA_QS(2); break;
    case 4: SA_QS(4); break;
    case 8: SA_QS(8); break;
    default: SA_QS(16); break;
  }
#undef SA_QS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quest_score(int kv_dtype, int q_dtype, const void* q, const void* meta,
                              const Shapes& s, const int32_t* pt, const int32_t* lens,
                              float* scores, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  dim3 grid((s.max_pages + kScorePagesPerWG - 1) / kScorePagesPerWG, s.Hkv, s.B);
  if (kv_dtype == SA_F32)
    return q_dtype == SA_F32 ? quest_dispatch_g<SA_F32, SA_F32>(G, grid, st, q, meta, s, pt, lens, scores)
                             : quest_dispatch_g<SA_F32, SA_BF16>(G, grid, st, q, meta, s, pt, lens, scores);
  return q_dtype == SA_F32 ? quest_dispatch_g<SA_BF16, SA_F32>(G, grid, st, q, meta, s, pt, lens, scores)
                           : quest_dispatch_g<SA_BF16, SA_BF16>(G, grid, st, q, meta, s, pt, lens, scores);
}

hipError_t launch_sals_score(int q_dtype, const void* q, const uint8_t* codes,
                             const uint16_t* scales, const float* proj, const Shapes& s,
                             const int32_t* pt, const int32_t* lens, int unit_tokens, float tau,
                             float* scores, int max_units, hipStream_t st) {
  const int upw = 8;
  dim3 grid((max_units + upw - 1) / upw, s.B);
  const float tl2 = tau * kLog2e;
  if (q_dtype == SA_F32)
    hipLaunchKernelGGL(sals_score_kernel<SA_F32>, grid, dim3(256), 0, st, q, s.Hq, codes, scales,
                       proj, s.num_pages, s.Hkv, pt, lens, s.max_pages, unit_tokens, tl2, scores,
                       max_units, upw);
  else
    hipLaunchKernelGGL(sals_score_kernel<SA_BF16>, grid, dim3(256), 0, st, q, s.Hq, codes, scales,
                       proj, s.num_pages, s.Hkv, pt, lens, s.max_pages, unit_tokens, tl2, scores,
                       max_units, upw);
  return hipGetLastError();
}

}  // namespace sa
