// sa_attn.hip - standalone split-K attention over the selected pages
// (sa_sparse_decode_attn) and the split merge, on the device code of
// sa_dev_attn.h: one workgroup per (split, kv-head, batch), then one
// workgroup per list rescales and sums its splits' partial records.
#include "sa_dev_attn.h"

namespace sa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kUnionMaxPages = kUnionPages;

// grid (nsplit, Hkv, B), block 256: one split of one (batch, kv-head) list
template <int KT, int QT, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ num_sel, int max_sel, int pps,
    int nsplit, float scale_log2, float* __restrict__ partials, int masked) {
  __shared__ AttnSmem<G> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(lens[b], max_pages);
  int cnt = (L + kPage - 1) / kPage;
  const int32_t* lst = nullptr;
  if (sel) {
    lst = sel + ((size_t)b * hkv + h) * max_sel;
    cnt = min(num_sel[(size_t)b * hkv + h], max_sel);
  }
  const int j0 = split * pps, j1 = min(j0 + pps, cnt);
  // the split's list entries are read together with the list length
  const int jcap = sel ? min(j0 + pps, max_sel) : -1;
  float* part = partials + (((size_t)b * hkv + h) * nsplit + split) * G * kPartStride;
  // four or more bf16 query heads per kv-head: scores on the matrix cores
  if constexpr (G >= 4 && QT == SA_BF16 && (KT == SA_BF16 || KT == SA_I8))
    attend_range_mfma<KT, G>(q, k, v, ks, vs, num_pages, hkv, b, h, pt + (size_t)b * max_pages, L,
                             lst, j0, j1, scale_log2, part, sm, jcap, masked != 0);
  else
    attend_range<KT, QT, G>(q, k, v, ks, vs, num_pages, hkv, b, h, pt + (size_t)b * max_pages, L,
                            lst, j0, j1, scale_log2, part, sm, nullptr, jcap, masked != 0);
}

// grid (Hkv, B), block 256: the union of the page lists of the G query heads
// of one (b, kv-head) list, for per-head selection read as one pass over the
// group's pages ([Quest] GQA section: each head's own pages, and the union
// the group then has to load).  Head g's list is sel row (b * Hkv + h) * G + g.
// The union is written ascending, each entry (head mask << 16) | logical
// page, with its length in ucount.  One 16-bit head mask per logical page in
// LDS (n <= kUnionMaxPages).
__global__ __launch_bounds__(kAttnThreads) void union_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ num_sel, int max_sel, int G,
    int hkv, const int32_t* __restrict__ lens, int max_pages, int32_t* __restrict__ ulist,
    int32_t* __restrict__ ucount, int umax) {
  __shared__ uint32_t masks[kUnionMaxPages / 2];
  __shared__ int s_wave[kAttnThreads / 64];
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = (clamp_len(lens[b], max_pages) + kPage - 1) / kPage;
  for (int i = threadIdx.x; i < (n + 1) / 2; i += kAttnThreads) masks[i] = 0u;
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const size_t row = ((size_t)b * hkv + h) * G + g;
    const int cnt = min(num_sel[row], max_sel);
    for (int j = threadIdx.x; j < cnt; j += kAttnThreads) {
      const int p = sel[row * max_sel + j];
      if (p >= 0 && p < n) atomicOr(&masks[p >> 1], (1u << g) << (16 * (p & 1)));
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* out = ulist + ((size_t)b * hkv + h) * umax;
  int base = 0;  // entries written so far (the same in every thread)
  for (int p0 = 0; p0 < n; p0 += kAttnThreads) {
    const int p = p0 + threadIdx.x;
    const uint32_t m = p < n ? (masks[p >> 1] >> (16 * (p & 1))) & 0xFFFFu : 0u;
    const uint64_t bal = __ballot(m != 0u);
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int off = base, total = 0;
    for (int w = 0; w < kAttnThreads / 64; ++w) {
      if (w < wave) off += s_wave[w];
      total += s_wave[w];
    }
    off += __popcll(bal & ((1ull << lane) - 1ull));
    if (m != 0u && off < umax) out[off] = (int32_t)((m << 16) | (uint32_t)p);
    base += total;
    __syncthreads();  // s_wave is rewritten by the next round
  }
  if (threadIdx.x == 0) ucount[(size_t)b * hkv + h] = min(base, umax);
}

// grid (G, Hkv, B), block 256: merge the splits of one query head of one list
// (two thread groups of 128 outputs, each folding half of the splits)
__global__ __launch_bounds__(kAttnThreads) void merge_kernel(const float* __restrict__ partials,
                                                            int hkv, int G, int nsplit,
                                                            float* __restrict__ out) {
  __shared__ float lds[3 * kAttnThreads];
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t list = (size_t)b * hkv + h;
  merge_list(partials + list * nsplit * G * kPartStride, nsplit, G,
             out + ((size_t)b * hkv * G + (size_t)h * G) * kHeadDim, lds, nullptr, g, 1);
}

template <int KT, int QT>
hipError_t attn_dispatch_g(int G, dim3 grid, hipStream_t st, const void* q, const void* k,
                           const void* v, const uint16_t* ks, const uint16_t* vs, const Shapes& s,
                           const int32_t* pt, const int32_t* lens, const int32_t* sel,
                           const int32_t* num_sel, int max_sel, const AttnPlan& plan,
                           float scale_log2, float* partials, int masked) {
#define SA_AT(GG)                                                                               \
  hipLaunchKernelGGL((attn_kernel<KT, QT, GG>), grid, dim3(kAttnThreads), 0, st, q, k, v, ks,   \
                     vs, s.num_pages, s.Hkv, pt, lens, s.max_pages, sel, num_sel, max_sel,      \
                     plan.pps, plan.nsplit, scale_log2, partials, masked)
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
  // Selected lists: about two workgroups per CU, each wave taking the same
  // whole number of pages.  Measured on the GQA, SALS and large workloads,
  // fewer and longer splits beat filling the CUs: every split pays the list,
  // page-table and query round trips once, and the merge reads one record per
  // split.  Past 16 pages per wave the pass is bound by bandwidth, and more
  // workgroups (about eight per CU) keep more bytes in flight.
  constexpr long kLatencyWGs = 512, kBandwidthWGs = 2048, kMaxLatencyPPS = 64;
  AttnPlan p{};
  p.list_len = list_len < 1 ? 1 : list_len;
  const long lists = (long)B * Hkv;
  const int G = Hq / Hkv;
  const long pages = lists * p.list_len;
  long pps = ((pages + kLatencyWGs - 1) / kLatencyWGs + 3) / 4 * 4;
  if (pps > kMaxLatencyPPS) pps = (pages + kBandwidthWGs - 1) / kBandwidthWGs;
  if (pps < 4) pps = 4;
  p.pps = (int)pps;
  p.nsplit = (p.list_len + p.pps - 1) / p.pps;
  p.partial_floats = (size_t)lists * p.nsplit * G * kPartStride;
  return p;
}

hipError_t launch_attention(int kv_dtype, int q_dtype, const void* q, const void* k,
                            const void* v, const uint16_t* k_scale, const uint16_t* v_scale,
                            const Shapes& s, const int32_t* pt, const int32_t* lens,
                            const int32_t* sel, const int32_t* num_sel, int max_sel,
                            const AttnPlan& plan, float softmax_scale, float* partials,
                            float* out, hipStream_t st, bool masked) {
  const int G = s.Hq / s.Hkv;
  const float sl2 = softmax_scale * kLog2e;
  dim3 grid(plan.nsplit, s.Hkv, s.B);
  hipError_t e;
#define SA_KQ(KT, QT)                                                                        \
  e = attn_dispatch_g<KT, QT>(G, grid, st, q, k, v, k_scale, v_scale, s, pt, lens, sel, num_sel, \
                              max_sel, plan, sl2, partials, masked ? 1 : 0)
  if (kv_dtype == SA_F32) {
    if (q_dtype == SA_F32) SA_KQ(SA_F32, SA_F32); else SA_KQ(SA_F32, SA_BF16);
  } else if (kv_dtype == SA_BF16) {
    if (q_dtype == SA_F32) SA_KQ(SA_BF16, SA_F32); else SA_KQ(SA_BF16, SA_BF16);
  } else {
    if (q_dtype == SA_F32) SA_KQ(SA_I8, SA_F32); else SA_KQ(SA_I8, SA_BF16);
  }
#undef SA_KQ
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(G, s.Hkv, s.B), dim3(kAttnThreads), 0, st, partials, s.Hkv,
                     G, plan.nsplit, out);
  return hipGetLastError();
}

hipError_t launch_union(const int32_t* sel, const int32_t* num_sel, int max_sel, const Shapes& s,
                        const int32_t* lens, int32_t* ulist, int32_t* ucount, int umax,
                        hipStream_t st) {
  hipLaunchKernelGGL(union_kernel, dim3(s.Hkv, s.B), dim3(kAttnThreads), 0, st, sel, num_sel,
                     max_sel, s.Hq / s.Hkv, s.Hkv, lens, s.max_pages, ulist, ucount, umax);
  return hipGetLastError();
}

}  // namespace sa
