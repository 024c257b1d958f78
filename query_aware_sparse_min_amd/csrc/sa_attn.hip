// sa_attn.hip - standalone split-K attention over the selected pages
// (sa_sparse_decode_attn) and the split merge, on the device code of
// sa_dev_attn.h: one workgroup per (split, kv-head, batch), then one
// workgroup per list rescales and sums its splits' partial records.
#include "sa_dev_attn.h"

namespace sa {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kUnionMaxPages = kUnionPages;
// split plan: about two workgroups per CU while a wave takes at most 16 pages,
// else about eight (bandwidth-bound)
constexpr long kLatencyWGs = 512, kBandwidthWGs = 2048, kMaxLatencyPPS = 64;

// Device-side split plan of a dense pass over sequences of uneven length
// ("SALS长序列推理优化", tiling algorithm for variable-length input: cut the
// rows into basic blocks priced by a cost model, and bound every core by the
// average cost).  The basic block is one page of one (b, kv-head) list, priced
// by its bytes.  The pages over all lists fix the pages per split as the host
// plan does for lists of one length (about two workgroups per CU while a wave
// takes 16 pages or fewer, else about eight), and each list is cut into
// max(1, ceil(pages / pps)) splits, so a short sequence no longer gets the
// splits of the longest one.  Tasks are numbered b-major, then kv-head, then
// split: the splits of a list are adjacent and so are its partial records.
// Every workgroup of the attention and of the merge derives the same plan from
// the lengths (one read of B words), so the plan needs no launch of its own and
// no table in memory.  On return pre[b] is the first task of sequence b,
// pre[B] the number of tasks and, if len_s is given, len_s[b] the clamped
// length of sequence b.  NT threads, B <= kPlanMaxSeqs; all threads call.
struct RaggedPlan {
  int pps, tasks;
};

template <int NT>
__device__ RaggedPlan ragged_plan(const int32_t* __restrict__ lens, int B, int max_pages, int hkv,
                                  int* pre, uint32_t* red, int* len_s = nullptr) {
  constexpr int NW = NT / 64, PER = kPlanMaxSeqs / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int pg[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {  // thread tid holds sequences PER * tid .. + PER - 1
    const int b = PER * tid + e;
    const int L = b < B ? clamp_len(lens[b], max_pages) : 0;
    if (len_s && b < B) len_s[b] = L;
    pg[e] = (L + kPage - 1) / kPage;
    sum += (uint32_t)pg[e];
  }
  uint32_t incl = wave_incl_scan_u32(sum);
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  uint64_t total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) total += red[w];
  total *= (uint64_t)hkv;  // pages over all lists
  uint64_t pps = ((total + kLatencyWGs - 1) / kLatencyWGs + 3) / 4 * 4;
  if (pps > kMaxLatencyPPS) pps = (total + kBandwidthWGs - 1) / kBandwidthWGs;
  if (pps < 4) pps = 4;
  uint32_t cnt = 0, sp[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int b = PER * tid + e;
    sp[e] = b < B ? (uint32_t)hkv * (uint32_t)max(1, (int)((pg[e] + pps - 1) / pps)) : 0u;
    cnt += sp[e];
  }
  incl = wave_incl_scan_u32(cnt);
  __syncthreads();  // every wave has read red
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  uint32_t off = incl - cnt, tasks = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) off += red[w];
    tasks += red[w];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int b = PER * tid + e;
    if (b < B) pre[b] = (int)off;
    off += sp[e];
  }
  if (tid == 0) pre[B] = (int)tasks;
  __syncthreads();
  return {(int)pps, (int)tasks};
}

// The sequence, kv-head and split of planned task t (< pre[B]).
__device__ __forceinline__ void ragged_task(const int* pre, int B, int hkv, int t, int& b, int& h,
                                            int& split) {
  int lo = 0, hi = B - 1;  // the last sequence whose first task is <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  b = lo;
  const int spl = (pre[b + 1] - pre[b]) / hkv, r = t - pre[b];
  h = r / spl;
  split = r % spl;
}

// One split of one (batch, kv-head) list: pages [split * pps, + pps) of the
// sequence (sel == nullptr) or of its selected list, into the partial records
// part[G][kPartStride].  MPW: pages per wave in flight with the matrix-core
// scores (2 for the long splits of the dense device plan).
template <int KT, int QT, int G, int MPW = 1>
__device__ __forceinline__ void attn_task(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs, int num_pages, int hkv,
    const int32_t* __restrict__ pt, int max_pages, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ num_sel, int max_sel, int b, int h, int split, int pps, int L,
    float scale_log2, float* __restrict__ part, int masked, AttnSmem<G>& sm) {
  int cnt = (L + kPage - 1) / kPage;
  const int32_t* lst = nullptr;
  if (sel) {
    lst = sel + ((size_t)b * hkv + h) * max_sel;
    cnt = min(num_sel[(size_t)b * hkv + h], max_sel);
  }
  const int j0 = split * pps, j1 = min(j0 + pps, cnt);
  // the split's list entries are read together with the list length
  const int jcap = sel ? min(j0 + pps, max_sel) : -1;
  // four or more bf16 query heads per kv-head: scores on the matrix cores
  // (sixteen heads: one page per wave in flight, for registers)
  if constexpr (G >= 4 && QT == SA_BF16 && (KT == SA_BF16 || KT == SA_I8))
    attend_range_mfma<KT, G, 4, (G <= 8 ? MPW : 1)>(q, k, v, ks, vs, num_pages, hkv, b, h,
                                                 pt + (size_t)b * max_pages, L, lst, j0, j1, scale_log2,
                                                 part, sm, jcap, masked != 0);
  else
    attend_range<KT, QT, G>(q, k, v, ks, vs, num_pages, hkv, b, h, pt + (size_t)b * max_pages, L,
                            lst, j0, j1, scale_log2, part, sm, nullptr, jcap, masked != 0);
}

// grid (nsplit, Hkv, B), block 256: one split of one (batch, kv-head) list.
// PLAN (dense passes only): grid (bound on the tasks), task blockIdx.x of the
// device plan above; workgroups past the plan's tasks return at once.  (Dealing
// the tasks round-robin over a grid of resident workgroups, so that each pays
// for the plan once, measured slower: the hardware's dynamic dispatch of
// one-task workgroups balances uneven workgroup times better.)
template <int KT, int QT, int G, bool PLAN>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ num_sel, int max_sel, int pps,
    int nsplit, float scale_log2, float* __restrict__ partials, int masked, int B) {
  __shared__ AttnSmem<G> sm;
  if constexpr (PLAN) {
    __shared__ int pre[kPlanMaxSeqs + 1], len_s[kPlanMaxSeqs];
    __shared__ uint32_t red[kAttnThreads / 64];
    const RaggedPlan rp = ragged_plan<kAttnThreads>(lens, B, max_pages, hkv, pre, red, len_s);
    const int t = blockIdx.x;
    if (t >= rp.tasks) return;
    int b, h, split;
    ragged_task(pre, B, hkv, t, b, h, split);
    attn_task<KT, QT, G, 2>(q, k, v, ks, vs, num_pages, hkv, pt, max_pages, sel, num_sel, max_sel, b, h,
                            split, rp.pps, len_s[b], scale_log2,
                            partials + (size_t)t * G * kPartStride, masked, sm);
  } else {
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    attn_task<KT, QT, G>(q, k, v, ks, vs, num_pages, hkv, pt, max_pages, sel, num_sel, max_sel, b, h,
                         split, pps, clamp_len(lens[b], max_pages), scale_log2,
                         partials + (((size_t)b * hkv + h) * nsplit + split) * G * kPartStride,
                         masked, sm);
  }
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
// (two thread groups of 128 outputs, each folding half of the splits).  PLAN:
// the list's splits and records come from the device plan of the attention.
template <bool PLAN>
__global__ __launch_bounds__(kAttnThreads) void merge_kernel(const float* __restrict__ partials,
                                                            int hkv, int G, int nsplit,
                                                            float* __restrict__ out,
                                                            const int32_t* __restrict__ lens, int B,
                                                            int max_pages) {
  __shared__ float lds[3 * kAttnThreads];
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  size_t first = ((size_t)b * hkv + h) * nsplit;
  int ns = nsplit;
  if constexpr (PLAN) {
    __shared__ int pre[kPlanMaxSeqs + 1];
    __shared__ uint32_t red[kAttnThreads / 64];
    ragged_plan<kAttnThreads>(lens, B, max_pages, hkv, pre, red);
    ns = (pre[b + 1] - pre[b]) / hkv;
    first = (size_t)pre[b] + (size_t)h * ns;
  }
  merge_list(partials + first * G * kPartStride, ns, G,
             out + ((size_t)b * hkv * G + (size_t)h * G) * kHeadDim, lds, g, 1);
}

template <int KT, int QT, bool PLAN>
hipError_t attn_dispatch_g(int G, dim3 grid, hipStream_t st, const void* q, const void* k,
                           const void* v, const uint16_t* ks, const uint16_t* vs, const Shapes& s,
                           const int32_t* pt, const int32_t* lens, const int32_t* sel,
                           const int32_t* num_sel, int max_sel, const AttnPlan& plan,
                           float scale_log2, float* partials, int masked) {
#define SA_AT(GG)                                                                               \
  hipLaunchKernelGGL((attn_kernel<KT, QT, GG, PLAN>), grid, dim3(kAttnThreads), 0, st, q, k, v, \
                     ks, vs, s.num_pages, s.Hkv, pt, lens, s.max_pages, sel, num_sel, max_sel,  \
                     plan.pps, plan.nsplit, scale_log2, partials, masked, s.B)
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

AttnPlan plan_attention(int B, int Hq, int Hkv, int list_len, bool dense) {
  // Selected lists: about two workgroups per CU, each wave taking the same
  // whole number of pages.  Measured on the GQA, SALS and large workloads,
  // fewer and longer splits beat filling the CUs: every split pays the list,
  // page-table and query round trips once, and the merge reads one record per
  // split.  Past 16 pages per wave the pass is bound by bandwidth, and more
  // workgroups (about eight per CU) keep more bytes in flight.
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
  p.tasks = 0;
  // a batch of one sequence has nothing to balance: the host plan is the same
  if (dense && B > 1 && B <= kPlanMaxSeqs) {
    // the device plan cuts the pages actually present: fewer than
    // min(kBandwidthWGs, pages / 4) + one per list tasks (see ragged_plan)
    const long bound = (pages / 4 < kBandwidthWGs ? pages / 4 : kBandwidthWGs) + lists + 1;
    p.tasks = (int)bound;
    const size_t pf = (size_t)bound * G * kPartStride;
    if (pf > p.partial_floats) p.partial_floats = pf;
  }
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
  const bool planned = sel == nullptr && plan.tasks > 0 && s.B <= kPlanMaxSeqs;
  const dim3 grid = planned ? dim3(plan.tasks) : dim3(plan.nsplit, s.Hkv, s.B);
  hipError_t e;
#define SA_KQ(KT, QT)                                                                          \
  e = planned ? attn_dispatch_g<KT, QT, true>(G, grid, st, q, k, v, k_scale, v_scale, s, pt, lens, \
                                              sel, num_sel, max_sel, plan, sl2, partials,        \
                                              masked ? 1 : 0)                                    \
              : attn_dispatch_g<KT, QT, false>(G, grid, st, q, k, v, k_scale, v_scale, s, pt,    \
                                               lens, sel, num_sel, max_sel, plan, sl2, partials, \
                                               masked ? 1 : 0)
  if (kv_dtype == SA_F32) {
    if (q_dtype == SA_F32) SA_KQ(SA_F32, SA_F32); else SA_KQ(SA_F32, SA_BF16);
  } else if (kv_dtype == SA_BF16) {
    if (q_dtype == SA_F32) SA_KQ(SA_BF16, SA_F32); else SA_KQ(SA_BF16, SA_BF16);
  } else {
    if (q_dtype == SA_F32) SA_KQ(SA_I8, SA_F32); else SA_KQ(SA_I8, SA_BF16);
  }
#undef SA_KQ
  if (e != hipSuccess) return e;
  if (planned)
    hipLaunchKernelGGL(merge_kernel<true>, dim3(G, s.Hkv, s.B), dim3(kAttnThreads), 0, st, partials,
                       s.Hkv, G, plan.nsplit, out, lens, s.B, s.max_pages);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3(G, s.Hkv, s.B), dim3(kAttnThreads), 0, st, partials,
                       s.Hkv, G, plan.nsplit, out, lens, s.B, s.max_pages);
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
