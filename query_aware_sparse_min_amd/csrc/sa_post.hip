// sa_post.hip - selection, attention and merge of a decode step in one
// persistent kernel, after a separate scorer ("SALS长序列推理优化": QSI's
// exact top-k feeds SFAA, whose rows are split over cores and reduced;
// "Quest 完全拆解": top-K filtering, then attention over the kept pages only;
// "SequenceO1" explainer, FlashSA: only integer indices pass from selection
// to attention).
//
// Every list (batch, kv-head) is served by nc chunk tasks.  Each task:
//   1. runs the exact top-K of the whole list from its scores (written by the
//      scorer kernel before this one started, so nothing is waited for), with
//      each kept unit's rank;
//   2. expands kept unit of rank r to page slots r*upu .. r*upu + upu - 1 and
//      takes the slots [c S / nc, (c + 1) S / nc) of the S = kept units * upu
//      slots (an equal share of the kept pages wherever they lie), writing
//      their entries of the optional page list;
//   3. resolves its pages through the page table (one round trip) and attends
//      to them: query-head group on the matrix cores for G >= 4, else on the
//      vector ALUs; stores its partial record device-coherently;
//   4. counts itself done on the list's arrival counter after its stores have
//      completed; the chunk that arrives last merges the list's records into
//      out and returns the counter to 0.
// No workgroup waits for another one, so any number of them may be resident.
#include "sa_dev_attn.h"
#include "sa_dev_topk.h"
#include "sa_post.h"

namespace sa {
namespace {

template <int G, int NW>
union PostSmem {
  TopkSmem<64 * NW> topk;
  AttnSmem<G, NW> attn;
  float merge[3 * 64 * NW];
};

// KPT: top-K keys per thread in registers.  MFMA: the group's scores on the matrix cores.  PW: pages per wave in
// flight.
template <int KT, int G, int NW, int KPT, bool MFMA, int PW>
__global__ __launch_bounds__(64 * NW, 1) void post_score_kernel(PostArgs A, PostPlan P) {
  constexpr int NT = 64 * NW;
  __shared__ PostSmem<G, NW> sm;
  __shared__ int32_t s_log[kPostMaxShare];   // logical page of each slot of the share, or -1
  __shared__ int32_t s_list[kPostMaxShare];  // resolved: (physical << 4) | (valid - 1), or -1
  __shared__ int s_last, s_lastkept;
  const int tid = threadIdx.x;
  const int hq = A.hkv * G;
  const int upu = A.unit_tokens / kPage;

  for (int t = blockIdx.x; t < P.n_tasks; t += gridDim.x) {
    const int i = t / P.nc, c = t % P.nc;
    const int b = i / A.hkv, h = i % A.hkv;
    const int32_t* pt_row = A.pt + (size_t)b * A.max_pages;
    const float* sc_row = A.scores + (size_t)i * A.max_units;
    const int L = clamp_len(A.lens[b], A.max_pages);
    const int n = (L + A.unit_tokens - 1) / A.unit_tokens;  // units
    const int np = (L + kPage - 1) / kPage;                 // pages
    const int kept = n <= A.n_head + A.n_tail + A.k_compete ? n : A.n_head + A.k_compete + A.n_tail;
    const int S = kept * upu;
    const int lo = (int)((long)c * S / P.nc), hi = (int)((long)(c + 1) * S / P.nc);
    int32_t* sel_row = A.sel ? A.sel + (size_t)i * A.max_sel : nullptr;
    if (tid == 0) s_lastkept = 0;
    for (int j = tid; j < hi - lo; j += NT) s_log[j] = -1;
    __syncthreads();

    // 1-2. the list's selection; this chunk's slots of the kept pages
    topk_core<NT, KPT, false>(sc_row, n, A.k_compete, A.n_head, A.n_tail, sm.topk, [&](int rank, int u) {
      if (u == n - 1) s_lastkept = 1;
      for (int e = 0; e < upu; ++e) {
        const int slot = rank * upu + e, p = u * upu + e;
        if (slot >= lo && slot < hi && p < np) {
          s_log[slot - lo] = p;
          if (sel_row && slot < A.max_sel) sel_row[slot] = p;
        }
      }
    }, true);
    __syncthreads();
    if (sel_row && c == 0) {  // count and padding of the optional page list
      const int cnt = min(s_lastkept ? S - (upu - (np - (n - 1) * upu)) : S, A.max_sel);
      for (int j = cnt + tid; j < A.max_sel; j += NT) sel_row[j] = -1;
      if (tid == 0) A.num_sel[i] = n > 0 ? cnt : 0;
    }
    // 3. the share's pages through the page table, then the attention
    for (int j = tid; j < hi - lo; j += NT) {
      const int p = s_log[j];
      int r = -1;
      if (p >= 0) {
        const int pp = pt_row[p];
        if (pp >= 0 && pp < A.num_pages) r = (pp << 4) | (min(kPage, L - p * kPage) - 1);
      }
      s_list[j] = r;
    }
    __syncthreads();
    float* part_list = A.partials + (size_t)i * P.nc * G * kPartStride;
    float* part = part_list + (size_t)c * G * kPartStride;
    if constexpr (MFMA)
      attend_range_mfma<KT, G, NW, PW, true>(A.q, A.k, A.v, A.ks, A.vs, A.num_pages, A.hkv, b, h, pt_row, L,
                                            nullptr, 0, hi - lo, A.scale_log2, part, sm.attn, -1, false,
                                            s_list);
    else
      attend_range<KT, SA_BF16, G, PW, true, NW>(A.q, A.k, A.v, A.ks, A.vs, A.num_pages, A.hkv, b, h, pt_row,
                                                 L, nullptr, 0, hi - lo, A.scale_log2, part, sm.attn,
                                                 s_list);
    // 4. arrival: every store of this task has completed before the count,
    // which wave 0 takes; the list's last chunk merges the list and returns the
    // counter to 0 (one or two query heads: wave 0 alone, measured faster;
    // more: the whole workgroup, whose groups fold the records in parallel)
    stores_done();
    __syncthreads();
    float* out_row = A.out + ((size_t)b * hq + (size_t)h * G) * kHeadDim;
    if constexpr (G <= 2) {
      if (tid < 64) {
        uint32_t prev = 0u;
        if (tid == 0) prev = __hip_atomic_fetch_add(A.arrive + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
        if (prev == (uint32_t)(P.nc - 1)) {
          merge_list_wave<G, true>(part_list, P.nc, out_row);
          if (tid == 0) st_x<true>(A.arrive + i, 0u);
        }
      }
    } else {
      if (tid == 0)
        s_last = __hip_atomic_fetch_add(A.arrive + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(P.nc - 1);
      __syncthreads();
      if (s_last) {
        merge_list<true, 4>(part_list, P.nc, G, out_row, sm.merge);
        if (tid == 0) st_x<true>(A.arrive + i, 0u);
      }
    }
    __syncthreads();  // shared memory is reused by the next task
  }
}

constexpr int kPostKpt = 4;  // register keys per thread for lists of up to 64 NW * 4 units

// Waves per workgroup within the register budget of the group's attention:
// eight waves for up to eight heads (at most 256 VGPRs), four for 16 (the
// 16-head accumulators take up to 512).
constexpr int post_waves(int G) { return G <= 8 ? 8 : 4; }
constexpr int post_threads(int G) { return 64 * post_waves(G); }

template <int KT, int G>
hipError_t post_dispatch(const PostArgs& A, const PostPlan& P, hipStream_t st) {
  constexpr int NW = post_waves(G);
  constexpr bool kMfma = G >= 4;
  constexpr int PW = G == 2 || G >= 16 ? 1 : 2;
  hipLaunchKernelGGL((post_score_kernel<KT, G, NW, kPostKpt, kMfma, PW>), dim3(P.grid), dim3(64 * NW), 0, st, A,
                     P);
  return hipGetLastError();
}

template <int KT>
hipError_t post_dispatch_g(int G, const PostArgs& A, const PostPlan& P, hipStream_t st) {
  switch (G) {
    case 1: return post_dispatch<KT, 1>(A, P, st);
    case 2: return post_dispatch<KT, 2>(A, P, st);
    case 4: return post_dispatch<KT, 4>(A, P, st);
    case 8: return post_dispatch<KT, 8>(A, P, st);
    default: return post_dispatch<KT, 16>(A, P, st);
  }
}

}  // namespace

bool post_supported(int kv_dtype, int q_dtype, int G, int max_units) {
  // every chunk task runs the list's whole top-K: only with its keys in
  // registers (longer lists keep the single top-K launch of the separate kernels)
  return q_dtype == SA_BF16 && (kv_dtype == SA_BF16 || kv_dtype == SA_I8) &&
         max_units <= post_threads(G) * kPostKpt;
}

PostPlan plan_post(int lists, int G, int kept_pages, int num_cus) {
  PostPlan P{};
  P.lists = lists;
  // about one task per compute unit, and no share longer than kPostMaxShare
  long nc = (num_cus + lists - 1) / lists;
  const long need = (kept_pages + kPostMaxShare - 1) / kPostMaxShare;
  if (nc < need) nc = need;
  if (nc > kPostMaxChunks) nc = kPostMaxChunks;
  if (nc < 1) nc = 1;
  P.nc = (int)nc;
  P.ok = (long)P.nc * kPostMaxShare >= kept_pages;
  P.n_tasks = lists * P.nc;
  P.grid = P.n_tasks < num_cus ? P.n_tasks : num_cus;
  (void)G;
  return P;
}

hipError_t launch_post_score(int kv_dtype, int G, const PostArgs& A, const PostPlan& P, hipStream_t st) {
  if (kv_dtype == SA_I8) return post_dispatch_g<SA_I8>(G, A, P, st);
  return post_dispatch_g<SA_BF16>(G, A, P, st);
}

}  // namespace sa
