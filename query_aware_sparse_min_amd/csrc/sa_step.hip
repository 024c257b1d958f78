// sa_step.hip - the whole Quest decode step as one persistent kernel.
//
// "SequenceO1" explainer (FlashSA): selection and sparse attention are two
// stages joined only by integer indices.  "Quest 完全拆解": criticality
// estimation, top-K filtering, then attention over the kept pages only.
//
// Every list (batch, kv-head) is cut into nc chunks of consecutive logical
// pages; one task per chunk does, in one workgroup:
//   1. score its pages (Quest bound) and store their order keys, with the
//      list's page-table row fetched alongside into LDS;
//   2. run the exact top-K of the whole list from all of its keys -- every
//      chunk of the list computes the same selection, with each kept page's
//      rank -- and take the kept pages of ranks [c K / nc, (c + 1) K / nc)
//      (K kept pages), an equal share wherever they lie in the list, resolved
//      through the row in LDS (writing their entries of the optional page
//      list at their ranks);
//   3. attend to those pages (online softmax) and store one partial record;
//   4. count itself done on the list's arrival counter; the chunk that
//      arrives last merges the list's nc partial records into out and returns
//      the list's keys and counter to 0.
// So only the scores cross between workgroups before the attention.
//
// No workgroup ever waits for another one, so the kernel is correct whatever
// subset of its grid is resident at a time:
//  - keys: every key word is nonzero once written (order keys), the workspace
//    holds zeros before the call, and a reader re-reads, device-coherently,
//    every word still 0 -- for a bounded time.  Keys still missing then are
//    computed by the reader itself: it scores the missing chunks with the same
//    device code, so the words it stores are bit-identical to the owner's, and
//    every chunk of the list sees the same keys whichever workgroup wrote them.
//  - partial records: each chunk stores its record device-coherently, waits
//    until the stores have completed, and only then increments the counter, so
//    the chunk that sees nc - 1 reads every record complete.  Its own key
//    stores have completed by then as well, so once the last chunk clears the
//    keys no late key store of this call can follow.
// Task t runs on workgroup t mod grid; the grid is about the number of
// workgroups the device holds at once (one per CU), so normally every chunk of
// a list is resident together and nobody computes another chunk's scores.
#include "sa_dev_score.h"
#include "sa_dev_topk.h"
#include "sa_step.h"

namespace sa {
namespace {

constexpr int kStepWaves = 8;               // one workgroup per CU: 8 waves, up to 256 VGPRs each
constexpr int kStepThreads = 64 * kStepWaves;
constexpr int kScoreIT = (64 + kStepWaves - 1) / kStepWaves;  // load pairs per lane per score pass
constexpr int kScorePass = 4 * kStepWaves * kScoreIT;          // pages per score pass (>= 256)
constexpr int kChunkGrain = 16;                                // chunk sizes are multiples of this

template <int G>
union StepSmem {
  TopkSmem<kStepThreads> topk;
  AttnSmem<G, kStepWaves> attn;
};

// Keys of a list that have not arrived in time: the chunks that hold them are
// scored again here (topk_core's help protocol).  mark() records the chunk of
// a missing unit in an LDS bit mask; run() scores every marked chunk with the
// same code the chunk's own task runs, stores the keys and waits for them.
template <typename ScoreChunk>
struct StepHelp {
  uint32_t* mask;  // LDS, one bit per chunk of the list
  int chunk_pages, nc;
  ScoreChunk score_chunk;
  __device__ __forceinline__ void mark(int u) const {
    const int c = u / chunk_pages;
    atomicOr(&mask[c >> 5], 1u << (c & 31));
  }
  __device__ __forceinline__ void run() const {
    for (int c = 0; c < nc; ++c)
      if ((mask[c >> 5] >> (c & 31)) & 1u) score_chunk(c);
    stores_done();
  }
};

// KPT: top-K keys per thread in registers (lists of up to kStepThreads * KPT pages).
// PW: pages each wave of the attention loads at once.
template <int KT, int QT, int G, int KPT, int PW>
__global__ __launch_bounds__(kStepThreads, 1) void quest_step_kernel(StepArgs A, StepPlan P) {
  static_assert(G == 1, "one query head per kv-head: the merge is one wave's");
  __shared__ StepSmem<G> sm;
  __shared__ int32_t s_pt[kStepThreads * KPT];   // the list's page-table row
  // this chunk's share of the kept pages: (physical << 4) | (valid - 1), or -1
  __shared__ int32_t s_list[kStepMaxChunk];
  __shared__ uint32_t s_help[kStepMaxPages / kChunkGrain / 32];  // chunks whose keys are missing
  const int tid = threadIdx.x;
  const int hq = A.hkv * G;

  for (int t = blockIdx.x; t < P.n_tasks; t += gridDim.x) {
    const int i = t / P.nc, c = t % P.nc;
    const int b = i / A.hkv, h = i % A.hkv;
    const int32_t* pt_row = A.pt + (size_t)b * A.max_pages;
    float* sc_row = A.scores + (size_t)i * A.max_pages;

    // scores of chunk cc stored as order keys, IT page pairs per lane and pass;
    // the passes cover the chunk up to the page-table row length, so their
    // loads need not wait for the sequence length.  A page's key does not
    // depend on IT (sixteen lanes of one row reduce it in a fixed order).
    // Returns the list's page count.
    auto score_chunk = [&](auto it_c, int cc) {
      constexpr int IT = decltype(it_c)::value, kPass = 4 * kStepWaves * IT;
      const int a0 = cc * P.chunk_pages, a1 = min(a0 + P.chunk_pages, A.max_pages);
      int nv = 0;
      for (int p0 = a0; p0 < a1; p0 += kPass)
        nv = quest_score_range<KT, QT, G, IT, true, kStepWaves, true>(
            A.q, A.meta, A.num_pages, A.hkv, b, h, pt_row, p0, min(p0 + kPass, a1), A.lens + b,
            A.max_pages, sc_row);
      return nv;
    };
    // the help path scores with one page pair per lane: fewer registers live
    // beside the selection's
    auto help_chunk = [&](int cc) { score_chunk(std::integral_constant<int, 1>{}, cc); };

    // 1. scores of the chunk; the list's page-table row (any kept page of the
    // list may fall to this chunk) goes out with the score loads and is parked
    // in LDS.  (fp32 metadata: half the page pairs per pass, for the register
    // budget.)
    int32_t ptv[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) ptv[r] = pt_row[min(tid + kStepThreads * r, A.max_pages - 1)];
    int n = score_chunk(std::integral_constant<int, KT == SA_F32 ? kScoreIT / 2 : kScoreIT>{}, c);
    const int L = clamp_len(A.lens[b], A.max_pages);
    if (c * P.chunk_pages >= A.max_pages) n = (L + kPage - 1) / kPage;
#pragma unroll
    for (int r = 0; r < KPT; ++r) s_pt[tid + kStepThreads * r] = ptv[r];
    for (int j = tid; j < (int)(sizeof(s_help) / sizeof(s_help[0])); j += kStepThreads) s_help[j] = 0u;
    // s_pt and the clears before the selection (the selection's own first
    // barrier would order them as well, but a common start of the waves' key
    // reads measured faster)
    __syncthreads();

    // 2. the list's selection (its keys re-read until all have arrived, or
    // scored here).  The kept pages are shared out by rank: chunk c attends to
    // the kept pages of ranks [lo, hi), an equal share whatever their place in
    // the list, resolved through the page-table row in LDS.
    const int kept = n <= A.n_head + A.n_tail + A.k_compete ? n : A.n_head + A.k_compete + A.n_tail;
    const int lo = (int)((long)c * kept / P.nc), hi = (int)((long)(c + 1) * kept / P.nc);
    int32_t* sel_row = A.sel ? A.sel + (size_t)i * A.max_sel : nullptr;
    const StepHelp<decltype(help_chunk)> help{s_help, P.chunk_pages, P.nc, help_chunk};
    topk_core<kStepThreads, KPT, true, true>(sc_row, n, A.k_compete, A.n_head, A.n_tail, sm.topk,
                                             [&](int rank, int u) {
                                               if (rank >= lo && rank < hi) {
                                                 const int pp = s_pt[u];
                                                 s_list[rank - lo] = (pp >= 0 && pp < A.num_pages)
                                                     ? (pp << 4) | (min(kPage, L - u * kPage) - 1) : -1;
                                                 if (sel_row && rank < A.max_sel) sel_row[rank] = u;
                                               }
                                             }, true, help);
    if (sel_row && c == 0) {  // count and padding of the optional page list
      const int cnt = min(kept, A.max_sel);
      for (int j = cnt + tid; j < A.max_sel; j += kStepThreads) sel_row[j] = -1;
      if (tid == 0) A.num_sel[i] = cnt;
    }
    __syncthreads();  // s_list complete

    // 3. attention over the chunk's share of the kept pages
    float* part_list = A.partials + (size_t)i * P.nc * G * kPartStride;
    attend_range<KT, QT, G, PW, true, kStepWaves, true>(A.q, A.k, A.v, nullptr, nullptr, A.num_pages, A.hkv, b,
                                                  h, pt_row, L, nullptr, 0, hi - lo, A.scale_log2,
                                                  part_list + (size_t)c * G * kPartStride, sm.attn, s_list);
    // 4. arrival: every store of this task has completed before the count,
    // which wave 0 takes (the other waves' stores completed before the
    // record's barrier, and wave 0 stored the record); if it is the list's
    // last chunk, wave 0 merges the list and returns its keys and counter to
    // 0.  The keys are next read in the next launch, so plain stores (16 bytes
    // per lane where the row allows) suffice: the launch boundary publishes them
    if (tid < 64) {
      stores_done();
      uint32_t prev = 0u;
      if (tid == 0) prev = __hip_atomic_fetch_add(A.arrive + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = (uint32_t)__builtin_amdgcn_readfirstlane((int)prev);
      if (prev == (uint32_t)(P.nc - 1)) {
        merge_list_wave<G, true>(part_list, P.nc, A.out + ((size_t)b * hq + (size_t)h * G) * kHeadDim);
        if (A.max_pages % 4 == 0) {
          uint4* kw = reinterpret_cast<uint4*>(sc_row);
          for (int j = tid; j < A.max_pages / 4; j += 64) kw[j] = make_uint4(0u, 0u, 0u, 0u);
        } else {
          uint32_t* kw = reinterpret_cast<uint32_t*>(sc_row);
          for (int j = tid; j < A.max_pages; j += 64) kw[j] = 0u;
        }
        if (tid == 0) st_x<true>(A.arrive + i, 0u);
      }
    }
    __syncthreads();  // shared memory is reused by the next task
  }
}

// register-resident top-K keys per thread: lists of up to kStepThreads * kKptLo pages, else kKptHi
constexpr int kKptLo = (2048 + kStepThreads - 1) / kStepThreads;
constexpr int kKptHi = (kStepMaxPages + kStepThreads - 1) / kStepThreads;

typedef void (*StepKernel)(StepArgs, StepPlan);

// two pages in flight per wave where the K/V rows are 16-bit (bf16): one round
// of loads covers a chunk's usual share; fp32 rows keep one (register budget)
template <int KT, int QT>
StepKernel step_kernel_of(int kpt) {
  constexpr int PW = KT == SA_BF16 ? 2 : 1;
  return kpt <= kKptLo ? quest_step_kernel<KT, QT, 1, kKptLo, PW> : quest_step_kernel<KT, QT, 1, kKptHi, PW>;
}

StepKernel kernel_of(int kv_dtype, int q_dtype, int kpt) {
  if (kv_dtype == SA_F32)
    return q_dtype == SA_F32 ? step_kernel_of<SA_F32, SA_F32>(kpt) : step_kernel_of<SA_F32, SA_BF16>(kpt);
  return q_dtype == SA_F32 ? step_kernel_of<SA_BF16, SA_F32>(kpt) : step_kernel_of<SA_BF16, SA_BF16>(kpt);
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

int step_kpt(int max_pages) { return max_pages <= kStepThreads * kKptLo ? kKptLo : kKptHi; }

int step_resident_wgs(int kv_dtype, int q_dtype, int kpt, int num_cus) {
  const StepKernel f = kernel_of(kv_dtype, q_dtype, kpt);
  // a build that spills keeps per-wave scratch, which the occupancy query does
  // not count and which can hold back waves: 0 then sends the step to the
  // separate kernels (the fused kernel would still be correct, but slow)
  hipFuncAttributes fa{};
  if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(f)) != hipSuccess || fa.localSizeBytes != 0)
    return 0;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kStepThreads, 0) != hipSuccess) return 0;
  return per_cu < 1 ? 0 : per_cu * num_cus;
}

hipError_t launch_quest_step(int kv_dtype, int q_dtype, const StepArgs& A, const StepPlan& P,
                             hipStream_t st) {
  hipLaunchKernelGGL(kernel_of(kv_dtype, q_dtype, step_kpt(A.max_pages)), dim3(P.grid), dim3(kStepThreads), 0,
                     st, A, P);
  return hipGetLastError();
}

}  // namespace sa
