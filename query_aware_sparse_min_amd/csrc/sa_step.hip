// sa_step.hip - the whole Quest decode step as one persistent kernel.
//
// "SequenceO1" explainer (FlashSA): selection and sparse attention are two
// stages joined only by integer indices.  "Quest 完全拆解": criticality
// estimation, top-K filtering, then attention over the kept pages only.
//
// Every list (batch, kv-head) is cut into nc chunks of consecutive logical
// pages; one task per chunk does, in one workgroup:
//   1. score its pages (Quest bound) and store their order keys, keeping the
//      chunk's physical page numbers in LDS;
//   2. run the exact top-K of the whole list from all of its keys -- every
//      chunk of the list computes the same selection -- and keep only the
//      selected pages of its own chunk (writing their entries of the optional
//      page list at their global ranks);
//   3. attend to those pages (online softmax) and store one partial record;
//   4. chunk 0 merges the list's nc partial records into out and clears the
//      list's keys and partials.
// So only the scores cross between workgroups before the attention, and the
// page table is read once per page.
//
// Hand-offs need no counters: every handed-off word is nonzero once written
// (order keys; partial words XOR a constant that no fp32 result takes), the
// workspace holds zeros before the call, and a reader re-reads, device-
// coherently, every word still 0 until all have arrived.  Stores are relaxed
// and device-coherent (sc1) and nobody waits for them to land.  Every re-read
// loop is bounded: on timeout ctl.error is set and the kernel still finishes.
// The keys and partials of a list are returned to 0 by its merger, which runs
// only after every chunk of the list has stored its partial record and so has
// finished reading keys.
//
// Scheduling: task t runs on workgroup t mod grid, in order; every workgroup
// is co-resident and grid >= nc.  A task waits only for the other chunks of
// its own list, which sit on other workgroups (nc <= grid) behind tasks of
// earlier lists only; the earliest unfinished list therefore always makes
// progress, and the schedule cannot deadlock.
#include "sa_dev_score.h"
#include "sa_dev_topk.h"
#include "sa_step.h"

namespace sa {
namespace {

constexpr int kStepWaves = 12;              // one workgroup per CU: 12 waves, 168 VGPRs each
constexpr int kStepThreads = 64 * kStepWaves;
constexpr int kScoreIT = (64 + kStepWaves - 1) / kStepWaves;  // load pairs per lane per score pass
constexpr int kScorePass = 4 * kStepWaves * kScoreIT;          // pages per score pass (>= 256)
constexpr int kChunkGrain = 16;                                // chunk sizes are multiples of this

template <int G>
union StepSmem {
  TopkSmem<kStepThreads> topk;
  AttnSmem<G, kStepWaves> attn;
  float merge[3 * kStepThreads];
};

// KPT: top-K keys per thread in registers (lists of up to 256 * KPT pages).
template <int KT, int QT, int G, int KPT>
__global__ __launch_bounds__(kStepThreads, 1) void quest_step_kernel(StepArgs A, StepPlan P) {
  __shared__ StepSmem<G> sm;
  __shared__ int32_t s_pp[kStepMaxChunk];    // physical page of each chunk page, or -1
  // chunk page kept by the selection: (physical << 4) | (valid - 1), else -1
  __shared__ int32_t s_kept[kStepMaxChunk];
  __shared__ int32_t s_list[kStepMaxChunk];  // kept pages: (physical << 4) | (valid - 1)
  __shared__ int s_cnt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hq = A.hkv * G;

  for (int t = blockIdx.x; t < P.n_tasks; t += gridDim.x) {
    const int i = t / P.nc, c = t % P.nc;
    const int b = i / A.hkv, h = i % A.hkv;
    const int32_t* pt_row = A.pt + (size_t)b * A.max_pages;
    const int c0 = c * P.chunk_pages;
    float* sc_row = A.scores + (size_t)i * A.max_pages;

    // 1. scores of the chunk; the passes cover the chunk up to the page-table
    // row length, so their loads need not wait for the sequence length
    const int c_end = min(c0 + P.chunk_pages, A.max_pages);
    int n = 0;
    for (int p0 = c0; p0 < c_end; p0 += kScorePass)
      n = quest_score_range<KT, QT, G, kScoreIT, true, kStepWaves, true>(A.q, A.meta, A.num_pages, A.hkv, b, h, pt_row,
                                                       p0, min(p0 + kScorePass, c_end), A.lens + b,
                                                       A.max_pages, sc_row, s_pp + (p0 - c0));
    const int L = clamp_len(A.lens[b], A.max_pages);
    if (c0 >= c_end) n = (L + kPage - 1) / kPage;
    const int c1 = min(c0 + P.chunk_pages, n);  // c1 <= c0: an empty chunk
    for (int j = tid; j < P.chunk_pages; j += kStepThreads) s_kept[j] = -1;
    __syncthreads();  // the clears (and s_pp) before the selection marks kept pages

    // 2. the list's selection (its keys re-read until all have arrived); keep this chunk's part
    int32_t* sel_row = A.sel ? A.sel + (size_t)i * A.max_sel : nullptr;
    topk_core<kStepThreads, KPT, true, true>(sc_row, n, A.k_compete, A.n_head, A.n_tail, sm.topk,
                                       [&](int rank, int u) {
                                         if (u >= c0 && u < c1) {
                                           const int pp = s_pp[u - c0];
                                           if (pp >= 0) s_kept[u - c0] = (pp << 4) | (min(kPage, L - u * kPage) - 1);
                                           if (sel_row && rank < A.max_sel) sel_row[rank] = u;
                                         }
                                       }, sel_row != nullptr, &A.ctl->error);
    if (sel_row && c == 0) {  // count and padding of the optional page list
      const int cnt = min(min(n, A.n_head + A.k_compete + A.n_tail), A.max_sel);
      for (int j = cnt + tid; j < A.max_sel; j += kStepThreads) sel_row[j] = -1;
      if (tid == 0) A.num_sel[i] = cnt;
    }
    __syncthreads();
    if (wave == 0) {  // kept pages of the chunk, ascending (four reads in flight per round)
      const int nch = c1 - c0;
      int cnt = 0;
      for (int base = 0; base < nch; base += 256) {
        int32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = base + 64 * q + lane;
          const int32_t x = s_kept[min(j, kStepMaxChunk - 1)];
          v[q] = j < nch ? x : -1;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint64_t bal = __ballot(v[q] >= 0);
          if (v[q] >= 0) s_list[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = v[q];
          cnt += __popcll(bal);
        }
      }
      if (lane == 0) s_cnt = cnt;
    }
    __syncthreads();

    // 3. attention over the chunk's kept pages
    float* part_list = A.partials + (size_t)i * P.nc * G * kPartStride;
    attend_range<KT, QT, G, 1, true, kStepWaves, true>(A.q, A.k, A.v, nullptr, nullptr, A.num_pages, A.hkv, b, h,
                                     pt_row, L, nullptr, 0, s_cnt, A.scale_log2,
                                     part_list + (size_t)c * G * kPartStride, sm.attn, s_list);
    // 4. chunk 0 merges the list's partial records as they arrive
    if (c == 0) {
      __syncthreads();  // the attention's shared memory is free before the merge reuses it
      merge_list<true, true, 4>(part_list, P.nc, G, A.out + ((size_t)b * hq + (size_t)h * G) * kHeadDim,
                             sm.merge, &A.ctl->error);
      // every chunk of this list has read the list's keys (before storing its
      // partial record): return keys and partials to the unwritten state (0)
      uint32_t* kw = reinterpret_cast<uint32_t*>(sc_row);
      for (int j = tid; j < A.max_pages; j += kStepThreads) st_x<true>(kw + j, 0u);
      uint32_t* pw = reinterpret_cast<uint32_t*>(part_list);
      for (int j = tid; j < P.nc * G * kPartStride; j += kStepThreads) st_x<true>(pw + j, 0u);
    }
    __syncthreads();  // shared memory is reused by the next task
  }
}

// register-resident top-K keys per thread: lists of up to kStepThreads * kKptLo pages, else kKptHi
constexpr int kKptLo = (2048 + kStepThreads - 1) / kStepThreads;
constexpr int kKptHi = (kStepMaxPages + kStepThreads - 1) / kStepThreads;

template <int KT, int QT>
hipError_t step_dispatch(int kpt, const StepArgs& A, const StepPlan& P, hipStream_t st) {
  if (kpt <= kKptLo)
    hipLaunchKernelGGL((quest_step_kernel<KT, QT, 1, kKptLo>), dim3(P.grid), dim3(kStepThreads), 0, st, A, P);
  else
    hipLaunchKernelGGL((quest_step_kernel<KT, QT, 1, kKptHi>), dim3(P.grid), dim3(kStepThreads), 0, st, A, P);
  return hipGetLastError();
}

template <int KT, int QT>
int resident_of(int kpt) {
  int per_cu = 0;
  const hipError_t e = kpt <= kKptLo
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quest_step_kernel<KT, QT, 1, kKptLo>, kStepThreads, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quest_step_kernel<KT, QT, 1, kKptHi>, kStepThreads, 0);
  return e == hipSuccess ? per_cu : 0;
}

}  // namespace

StepPlan plan_step(int B, int Hq, int Hkv, int max_pages, int max_sel, int num_cus) {
  StepPlan P{};
  (void)Hq;
  (void)max_sel;
  P.lists = B * Hkv;
  const long lists = P.lists;
  const long wgs = num_cus;  // resident workgroups aimed for: one per CU
  // chunks: about one per resident workgroup overall, in multiples of kChunkGrain pages
  long chunk = (lists * max_pages + wgs - 1) / wgs;
  chunk = (chunk + kChunkGrain - 1) / kChunkGrain * kChunkGrain;
  if (chunk < kChunkGrain) chunk = kChunkGrain;
  if (chunk > kStepMaxChunk) chunk = kStepMaxChunk;
  P.chunk_pages = (int)chunk;
  P.nc = (int)((max_pages + chunk - 1) / chunk);
  P.n_tasks = (int)(lists * P.nc);
  P.grid = (int)(wgs < P.n_tasks ? wgs : P.n_tasks);
  return P;
}

size_t step_ctl_bytes() { return sizeof(StepCtl); }

int step_kpt(int max_pages) { return max_pages <= kStepThreads * kKptLo ? kKptLo : kKptHi; }

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
