// sa_step.hip - the whole Quest decode step as one persistent kernel.
//
// "SequenceO1" explainer (FlashSA): selection and sparse attention are two
// stages joined only by integer indices; fusing them into one monolithic
// kernel cut occupancy.  Here the stages stay separate tasks with their own
// register/LDS shapes but run inside one launch ("Quest 完全拆解":
// criticality estimation, top-K filtering, approximate attention; only page
// numbers cross), so no stage waits for a kernel boundary.
//
// Task order: every score chunk (list-major), then every attention split
// (list-major).  The grid is sized to be co-resident and workgroup w runs
// tasks w, w + grid, w + 2 grid, ... in order.  A task waits only for tasks
// earlier in the order; the earliest unfinished task is always running (all
// workgroups are resident and each runs its tasks in order), so the schedule
// cannot deadlock.  Hand-offs use device-coherent (sc1) data stores, a wait
// for their completion, then a relaxed counter:
//   score chunk -> scores, then score_done[list] += 1; the chunk that brings
//                  score_done to the chunk count runs the list's top-K at once
//                  (also resolving the kept pages through the page table) and
//                  publishes the page lists with sel_ready = 1;
//   attention   -> waits sel_ready; partial record, then attn_done += 1; the
//                  split that brings attn_done to the split count merges the
//                  list's partials into out and clears the list's counters.
// Every wait is bounded: on timeout ctl.error is set and the kernel still
// finishes.  Control words live at the head of the caller's workspace: zero
// before the first call, and every call leaves them zero again.
#include "sa_dev_score.h"
#include "sa_dev_topk.h"
#include "sa_step.h"

namespace sa {
namespace {

constexpr int kStepThreads = 256;
constexpr int kScoreIT = 8;               // loads per lane per score pass
constexpr int kScorePass = 8 * kScoreIT;  // pages per score pass (64)
constexpr uint32_t kSpinLimit = 1u << 18;  // ~0.3 s of polling (each poll is a memory round trip)

// Thread 0 waits until *p >= target; the workgroup then continues.
__device__ __forceinline__ void wait_at_least(const uint32_t* p, uint32_t target, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (ld_x<true>(p) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Every thread's hand-off stores have completed; then thread 0 bumps *ctr.
__device__ __forceinline__ uint32_t publish_add(uint32_t* ctr) {
  stores_done();
  __syncthreads();
  uint32_t old = 0;
  if (threadIdx.x == 0)
    old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

template <int KT, int QT, int G>
union StepSmem {
  TopkSmem<kStepThreads> topk;
  AttnSmem<G> attn;
};

// KPT: top-K keys per thread in registers (lists of up to 256 * KPT pages).
template <int KT, int QT, int G, int KPT>
__global__ __launch_bounds__(kStepThreads, 4) void quest_step_kernel(StepArgs A, StepPlan P) {
  __shared__ StepSmem<KT, QT, G> sm;
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int hq = A.hkv * G;
  const int n_score = P.lists * P.nc;

  for (int t = blockIdx.x; t < P.n_tasks; t += gridDim.x) {
    const bool scoring = t < n_score;
    const int i = scoring ? t / P.nc : (t - n_score) / P.ns;
    const int idx = scoring ? t % P.nc : (t - n_score) % P.ns;
    const int b = i / A.hkv, h = i % A.hkv;
    ListCtl* lc = A.lctl + i;
    const int L = clamp_len(A.lens[b], A.max_pages);
    const int n = (L + kPage - 1) / kPage;
    const int32_t* pt_row = A.pt + (size_t)b * A.max_pages;

    if (scoring) {  // ------------------------------------- score chunk (+ top-K)
      const int c0 = idx * P.chunk_pages;
      const int c1 = min(c0 + P.chunk_pages, n);
      float* sc_row = A.scores + (size_t)i * A.max_pages;
      for (int p0 = c0; p0 < c1; p0 += kScorePass)
        quest_score_range<KT, QT, G, kScoreIT, true>(A.q, A.meta, A.num_pages, A.hkv, b, h, pt_row,
                                                     p0, min(p0 + kScorePass, c1), sc_row);
      const uint32_t old = publish_add(&lc->score_done);
      if (tid == 0) s_flag = old == (uint32_t)(P.nc - 1);
      __syncthreads();
      if (s_flag) {  // the list's last chunk: every score is in, select now
        topk_list<kStepThreads, KPT, true>(sc_row, n, n, 1, A.k_compete, A.n_head, A.n_tail,
                                                A.sel + (size_t)i * A.max_sel, A.num_sel + i,
                                                A.max_sel, sm.topk, pt_row, L, A.num_pages,
                                                A.rsel + (size_t)i * A.max_sel);
        publish_add(&lc->sel_ready);
      }
    } else {  // -------------------------------------------------------- attention split
      wait_at_least(&lc->sel_ready, 1u, &A.ctl->error);
      const int cnt = min(ld_x<true>(A.num_sel + i), A.max_sel);
      const int j0 = idx * P.pps, j1 = min(j0 + P.pps, cnt);
      float* part_list = A.partials + (size_t)i * P.ns * G * kPartStride;
      attend_range<KT, QT, G, 1, true>(A.q, A.k, A.v, nullptr, nullptr, A.num_pages, A.hkv, b, h,
                                       pt_row, L, A.sel + (size_t)i * A.max_sel, j0, j1,
                                       A.scale_log2, part_list + (size_t)idx * G * kPartStride,
                                       sm.attn, A.rsel + (size_t)i * A.max_sel);
      const uint32_t old = publish_add(&lc->attn_done);
      if (tid == 0) s_flag = old == (uint32_t)(P.ns - 1);
      __syncthreads();
      if (s_flag) {
        merge_list<true>(part_list, P.ns, G, A.out + ((size_t)b * hq + (size_t)h * G) * kHeadDim);
        if (tid == 0) {  // every task of this list has finished: clear its counters
          st_x<true>(&lc->score_done, 0u);
          st_x<true>(&lc->sel_ready, 0u);
          st_x<true>(&lc->attn_done, 0u);
        }
      }
    }
    __syncthreads();  // shared memory and s_flag are reused by the next task
  }
}

template <int KT, int QT>
hipError_t step_dispatch(int kpt, const StepArgs& A, const StepPlan& P, hipStream_t st) {
  if (kpt <= 8)
    hipLaunchKernelGGL((quest_step_kernel<KT, QT, 1, 8>), dim3(P.grid), dim3(kStepThreads), 0, st, A, P);
  else
    hipLaunchKernelGGL((quest_step_kernel<KT, QT, 1, 16>), dim3(P.grid), dim3(kStepThreads), 0, st, A, P);
  return hipGetLastError();
}

template <int KT, int QT>
int resident_of(int kpt) {
  int per_cu = 0;
  const hipError_t e = kpt <= 8
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quest_step_kernel<KT, QT, 1, 8>, kStepThreads, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quest_step_kernel<KT, QT, 1, 16>, kStepThreads, 0);
  return e == hipSuccess ? per_cu : 0;
}

}  // namespace

StepPlan plan_step(int B, int Hq, int Hkv, int max_pages, int max_sel, int num_cus) {
  StepPlan P{};
  P.lists = B * Hkv;
  const long lists = P.lists;
  (void)Hq;
  const long wgs = (long)num_cus * 4;  // resident workgroups aimed for
  // score chunks: about one per resident workgroup overall, whole passes of 64 pages
  long chunk = (lists * max_pages + wgs - 1) / wgs;
  chunk = (chunk + kScorePass - 1) / kScorePass * kScorePass;
  if (chunk < kScorePass) chunk = kScorePass;
  P.chunk_pages = (int)chunk;
  P.nc = (int)((max_pages + chunk - 1) / chunk);
  // attention splits: about one per resident workgroup, >= 4 pages (one per wave)
  long pps = (lists * max_sel + wgs - 1) / wgs;
  if (pps < 4) pps = 4;
  P.pps = (int)pps;
  P.ns = (int)((max_sel + pps - 1) / pps);
  P.n_tasks = (int)(lists * (P.nc + P.ns));
  P.grid = (int)(wgs < P.n_tasks ? wgs : P.n_tasks);
  return P;
}

size_t step_ctl_bytes(int lists) { return sizeof(StepCtl) + (size_t)lists * sizeof(ListCtl); }

int step_kpt(int max_pages) { return max_pages <= kStepThreads * 8 ? 8 : 16; }

int step_resident_wgs(int kv_dtype, int q_dtype, int kpt, int num_cus) {
  int per_cu;
  if (kv_dtype == SA_F32)
    per_cu = q_dtype == SA_F32 ? resident_of<SA_F32, SA_F32>(kpt) : resident_of<SA_F32, SA_BF16>(kpt);
  else
    per_cu = q_dtype == SA_F32 ? resident_of<SA_BF16, SA_F32>(kpt) : resident_of<SA_BF16, SA_BF16>(kpt);
  return per_cu < 1 ? 0 : per_cu * num_cus;
}

hipError_t launch_quest_step(int kv_dtype, int q_dtype, const StepArgs& A, const StepPlan& P,
                             hipStream_t st) {
  const int kpt = step_kpt(A.max_pages);
  if (kv_dtype == SA_F32)
    return q_dtype == SA_F32 ? step_dispatch<SA_F32, SA_F32>(kpt, A, P, st)
                             : step_dispatch<SA_F32, SA_BF16>(kpt, A, P, st);
  return q_dtype == SA_F32 ? step_dispatch<SA_BF16, SA_F32>(kpt, A, P, st)
                           : step_dispatch<SA_BF16, SA_BF16>(kpt, A, P, st);
}

}  // namespace sa
