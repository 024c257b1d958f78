// sa_step.h - plan, control words and launcher of the fused decode-step kernel.
#pragma once

#include "sa_internal.h"

namespace sa {

// Query heads per kv-head the fused kernel is built for (larger groups run
// the separate scorer / top-K / attention kernels).
constexpr int kStepMaxGroup = 1;
constexpr int kStepMaxPages = 4096;          // top-K keys of a list stay in registers
constexpr int kStepMaxPhysPages = 1 << 27;   // resolved pages pack the page id in 27 bits
constexpr int kStepMaxChunk = 1024;          // pages per chunk task (kept in LDS)

struct StepPlan {
  int lists;        // B * Hkv
  int chunk_pages;  // pages per chunk task (multiple of 16, <= kStepMaxChunk)
  int nc;           // chunk tasks per list
  int n_tasks;      // lists * nc
  int grid;         // workgroups launched (about the resident count; any value >= 1 is correct)
};

struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* meta;
  const int32_t* pt;
  const int32_t* lens;
  int B, hq, hkv, num_pages, max_pages;
  int k_compete, n_head, n_tail;
  float scale_log2;
  float* scores;    // [lists][max_pages]
  int32_t* sel;     // [lists][max_sel], optional
  int32_t* num_sel; // [lists], optional (given with sel)
  int max_sel;
  float* partials;  // [lists][nc][G][kHeadDim + 2]
  float* out;       // [B][hq][kHeadDim]
  uint32_t* arrive; // [lists] chunks of the list done so far (0 between calls)
};

StepPlan plan_step(int B, int Hq, int Hkv, int max_pages, int max_sel, int num_cus);
// Workgroups of the fused kernel that fit on the device at once (0 on error,
// or when the build uses scratch memory: the separate kernels run instead).
int step_resident_wgs(int kv_dtype, int q_dtype, int kpt, int num_cus);
// Top-K keys per thread of the fused kernel for lists of up to max_pages pages.
int step_kpt(int max_pages);
hipError_t launch_quest_step(int kv_dtype, int q_dtype, const StepArgs& A, const StepPlan& P,
                             hipStream_t st);

}  // namespace sa
