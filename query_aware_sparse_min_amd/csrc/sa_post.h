// sa_post.h - plan, arguments and launcher of the persistent selection +
// attention + merge kernel that follows a separate scorer.
#pragma once

#include "sa_internal.h"

namespace sa {

constexpr int kPostMaxShare = 512;   // kept pages one chunk task attends to, at most
constexpr int kPostMaxChunks = 256;  // chunk tasks per list, at most

struct PostPlan {
  int lists;    // B * Hkv
  int nc;       // chunk tasks per list
  int n_tasks;  // lists * nc
  int grid;     // workgroups launched (any value >= 1 gives the same result)
  bool ok;      // the kept pages of a list fit in nc shares
};

struct PostArgs {
  const void* q;            // bf16 [B][hq][d]
  const void* k;
  const void* v;
  const uint16_t* ks;       // int8 caches: fp16 scales
  const uint16_t* vs;
  const int32_t* pt;
  const int32_t* lens;
  int hkv, num_pages, max_pages;
  int unit_tokens, max_units;
  int k_compete, n_head, n_tail;
  float scale_log2;
  const float* scores;      // [lists][max_units], complete before the launch
  int32_t* sel;             // [lists][max_sel], optional
  int32_t* num_sel;         // [lists], optional (given with sel)
  int max_sel;
  float* partials;          // [lists][nc][G][kHeadDim + 2]
  float* out;               // [B][hq][kHeadDim]
  uint32_t* arrive;         // [lists] chunks done so far (0 between calls)
};

// bf16 query with a bf16 or int8 cache and lists whose top-K keys fit in the
// workgroup's registers (other steps use the separate kernels)
bool post_supported(int kv_dtype, int q_dtype, int G, int max_units);
PostPlan plan_post(int lists, int G, int kept_pages, int num_cus);
hipError_t launch_post_score(int kv_dtype, int G, const PostArgs& A, const PostPlan& P, hipStream_t st);

}  // namespace sa
