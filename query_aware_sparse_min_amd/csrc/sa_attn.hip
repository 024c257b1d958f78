// sa_attn.hip - flash-decoding attention over the selected pages (step 3)
// and the split merge.
//
// "Quest 完全拆解": approximate attention loads only the top-K pages, addressed
// through the page table.  "SALS长序列推理优化", SFAA: QK -> online softmax ->
// P@V -> rescale on int8 K/V gathered by the selection, with rows split across
// cores and reduced afterwards.  "Day 10·2": the softmax is renormalised over
// the selected set only.
//
// One workgroup = one (batch, kv-head, split).  Its four waves take the
// split's pages in turn; within a wave, lane l owns token row (l / 16) of a
// 4-row group and dimensions 8*(l % 16) .. +7, so each K/V load instruction
// reads four whole 256-byte rows (bf16) of the page.  Scores live in the
// base-2 domain (z = q.k * softmax_scale * log2 e); each wave keeps its own
// (max, sum, acc) per query head and the workgroup folds its four waves
// through LDS into one fp32 partial (acc[d], max, sum).  The merge kernel
// rescales the partials of all splits: out = sum acc_s 2^(m_s - M) /
// sum l_s 2^(m_s - M).
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kPartStride = kHeadDim + 2;  // acc[d], max, sum

// grid (nsplit, Hkv, B), block 256
template <int KT, int QT, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_valu_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ num_sel, int max_sel, int pps,
    int nsplit, float scale_log2, float* __restrict__ partials) {
  __shared__ float s_acc[4][G][kHeadDim];
  __shared__ float s_m[4][G], s_l[4][G];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int hq = hkv * G;
  const int L = clamp_len(lens[b], max_pages);
  const int np = (L + kPage - 1) / kPage;
  int cnt = np;
  const int32_t* lst = nullptr;
  if (sel) {
    lst = sel + ((size_t)b * hkv + h) * max_sel;
    cnt = min(num_sel[(size_t)b * hkv + h], max_sel);
  }
  const int j0 = split * pps, j1 = min(j0 + pps, cnt);

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

  for (int j = j0 + wave; j < j1; j += 4) {
    const int p = lst ? lst[j] : j;
    if (p < 0 || p >= np) continue;
    const int pp = pt[(size_t)b * max_pages + p];
    if (pp < 0 || pp >= num_pages) continue;
    const int nv = min(kPage, L - p * kPage);
    float kx[4][8], vx[4][8], ksc[4], vsc[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const size_t tok = ((size_t)pp * kPage + 4 * it + r) * hkv + h;
      load8<KT>(k, tok * kHeadDim + 8 * c, kx[it]);
      load8<KT>(v, tok * kHeadDim + 8 * c, vx[it]);
      if constexpr (KT == SA_I8) {
        ksc[it] = f16_to_f32(ks[tok]);
        vsc[it] = f16_to_f32(vs[tok]);
      } else {
        ksc[it] = vsc[it] = 1.0f;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float z[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qv[g][e], kx[it][e], s);
        s = xor_sum<1>(s);
        s = xor_sum<2>(s);
        s = xor_sum<4>(s);
        s = xor_sum<8>(s);
        z[it] = (4 * it + r < nv) ? s * (scale_log2 * ksc[it]) : -INFINITY;
      }
      float pm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      pm = xor_max<16>(pm);
      pm = xor_max<32>(pm);
      const float mn = fmaxf(m[g], pm);  // finite: slot 0 of a selected page is valid
      const float alpha = exp2f(m[g] - mn);
      float pr[4], psum = 0.0f;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        pr[it] = exp2f(z[it] - mn);
        psum += pr[it];
        pr[it] *= vsc[it];
      }
      l[g] = l[g] * alpha + psum;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = acc[g][e] * alpha;
#pragma unroll
        for (int it = 0; it < 4; ++it) a = fmaf(pr[it], vx[it][e], a);
        acc[g][e] = a;
      }
      m[g] = mn;
    }
  }

  // fold the four token rows of the wave, then the four waves of the workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = xor_sum<32>(xor_sum<16>(l[g]));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = xor_sum<32>(xor_sum<16>(acc[g][e]));
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][g][8 * c + e] = acc[g][e];
      if (c == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  float* part = partials + (((size_t)b * hkv + h) * nsplit + split) * G * kPartStride;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kAttnThreads) {
    const int g = idx / kHeadDim, dim = idx % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
    float a = 0.0f, ls = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(s_m[w][g] - M);
        a = fmaf(s_acc[w][g][dim], f, a);
        ls = fmaf(s_l[w][g], f, ls);
      }
    }
    part[g * kPartStride + dim] = a;
    if (dim == 0) {
      part[g * kPartStride + kHeadDim] = M;
      part[g * kPartStride + kHeadDim + 1] = ls;
    }
  }
}

// grid (Hq, B), block 128.  The (max, sum) pairs of all splits are fetched in
// parallel into LDS first, so the accumulator loads below are independent.
constexpr int kMergeMaxSplits = 1024;
__global__ __launch_bounds__(kHeadDim) void merge_kernel(const float* __restrict__ partials,
                                                         int hkv, int G, int nsplit,
                                                         float* __restrict__ out) {
  __shared__ float s_w[kMergeMaxSplits];
  __shared__ float s_red[2];
  const int hq_i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int h = hq_i / G, g = hq_i % G;
  const float* base = partials + ((size_t)b * hkv + h) * nsplit * G * kPartStride + g * kPartStride;
  const size_t stride = (size_t)G * kPartStride;
  // pass 1: per-thread max over its splits, then block max
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += kHeadDim) {
    const float ls = base[s * stride + kHeadDim + 1];
    const float ms = base[s * stride + kHeadDim];
    s_w[s] = ls;
    if (ls > 0.0f) M = fmaxf(M, ms);
  }
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(s_red[0], s_red[1]);
  // pass 2: weights 2^(m_s - M) (0 for empty splits) and the weighted sum of l
  for (int s = tid; s < nsplit; s += kHeadDim) {
    const float ls = s_w[s];
    s_w[s] = ls > 0.0f ? exp2f(base[s * stride + kHeadDim] - M) : 0.0f;
  }
  __syncthreads();
  float a = 0.0f, lsum = 0.0f;
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    const float a0 = base[(s + 0) * stride + tid], a1 = base[(s + 1) * stride + tid];
    const float a2 = base[(s + 2) * stride + tid], a3 = base[(s + 3) * stride + tid];
    const float l0 = base[(s + 0) * stride + kHeadDim + 1], l1 = base[(s + 1) * stride + kHeadDim + 1];
    const float l2 = base[(s + 2) * stride + kHeadDim + 1], l3 = base[(s + 3) * stride + kHeadDim + 1];
    const float w0 = s_w[s], w1 = s_w[s + 1], w2 = s_w[s + 2], w3 = s_w[s + 3];
    if (w0 > 0.0f) { a = fmaf(a0, w0, a); lsum = fmaf(l0, w0, lsum); }
    if (w1 > 0.0f) { a = fmaf(a1, w1, a); lsum = fmaf(l1, w1, lsum); }
    if (w2 > 0.0f) { a = fmaf(a2, w2, a); lsum = fmaf(l2, w2, lsum); }
    if (w3 > 0.0f) { a = fmaf(a3, w3, a); lsum = fmaf(l3, w3, lsum); }
  }
  for (; s < nsplit; ++s) {
    const float w = s_w[s];
    if (w > 0.0f) {
      a = fmaf(base[s * stride + tid], w, a);
      lsum = fmaf(base[s * stride + kHeadDim + 1], w, lsum);
    }
  }
  out[((size_t)b * hkv * G + hq_i) * kHeadDim + tid] = lsum > 0.0f ? a / lsum : 0.0f;
}

template <int KT, int QT>
hipError_t attn_dispatch_g(int G, dim3 grid, hipStream_t st, const void* q, const void* k,
                           const void* v, const uint16_t* ks, const uint16_t* vs, const Shapes& s,
                           const int32_t* pt, const int32_t* lens, const int32_t* sel,
                           const int32_t* num_sel, int max_sel, const AttnPlan& plan,
                           float scale_log2, float* partials) {
#define SA_AT(GG)                                                                               \
  hipLaunchKernelGGL((attn_valu_kernel<KT, QT, GG>), grid, dim3(kAttnThreads), 0, st, q, k, v,  \
                     ks, vs, s.num_pages, s.Hkv, pt, lens, s.max_pages, sel, num_sel, max_sel,  \
                     plan.pps, plan.nsplit, scale_log2, partials)
  switch (G) {
    case 1: SA_AT(1); break;
    case 2: SA_AT(2); break;
    case 4: SA_AT(4); break;
    case 8: SA_AT(8); break;
    default: SA_AT(16); break;
  }
#undef SA_AT
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attention(int B, int Hq, int Hkv, int list_len) {
  // Enough workgroups to cover the 256 CUs several times over; at least one
  // page per wave of a split.
  constexpr long kTargetWGs = 2048;
  AttnPlan p{};
  p.list_len = list_len < 1 ? 1 : list_len;
  const long lists = (long)B * Hkv;
  long pps = (lists * p.list_len + kTargetWGs - 1) / kTargetWGs;
  if (pps < 4) pps = 4;
  // the merge keeps one weight per split in LDS
  const long min_pps = (p.list_len + 1023) / 1024;
  if (pps < min_pps) pps = min_pps;
  p.pps = (int)pps;
  p.nsplit = (p.list_len + p.pps - 1) / p.pps;
  p.partial_floats = (size_t)lists * p.nsplit * (Hq / Hkv) * kPartStride;
  return p;
}

hipError_t launch_attention(int kv_dtype, int q_dtype, const void* q, const void* k,
                            const void* v, const uint16_t* k_scale, const uint16_t* v_scale,
                            const Shapes& s, const int32_t* pt, const int32_t* lens,
                            const int32_t* sel, const int32_t* num_sel, int max_sel,
                            const AttnPlan& plan, float softmax_scale, float* partials,
                            float* out, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  const float sl2 = softmax_scale * kLog2e;
  dim3 grid(plan.nsplit, s.Hkv, s.B);
  hipError_t e;
#define SA_KQ(KT, QT)                                                                        \
  e = attn_dispatch_g<KT, QT>(G, grid, st, q, k, v, k_scale, v_scale, s, pt, lens, sel, num_sel, \
                              max_sel, plan, sl2, partials)
  if (kv_dtype == SA_F32) {
    if (q_dtype == SA_F32) SA_KQ(SA_F32, SA_F32); else SA_KQ(SA_F32, SA_BF16);
  } else if (kv_dtype == SA_BF16) {
    if (q_dtype == SA_F32) SA_KQ(SA_BF16, SA_F32); else SA_KQ(SA_BF16, SA_BF16);
  } else {
    if (q_dtype == SA_F32) SA_KQ(SA_I8, SA_F32); else SA_KQ(SA_I8, SA_BF16);
  }
#undef SA_KQ
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(s.Hq, s.B), dim3(kHeadDim), 0, st, partials, s.Hkv, G,
                     plan.nsplit, out);
  return hipGetLastError();
}

}  // namespace sa
