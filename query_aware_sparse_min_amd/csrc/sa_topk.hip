// sa_topk.hip - standalone exact top-K (sa_topk_pages): one workgroup of 1024
// threads per (batch, kv-head) list running topk_list of sa_dev_topk.h, with
// 4 register keys per thread for lists of up to 4096 units and 16 for up to
// 16384 (more threads per list: shorter atomic and scan passes, measured
// 2.4-3.4 us faster than 256 threads x 16 keys on 2048-unit lists).
#include "sa_dev_topk.h"

namespace sa {
namespace {


// grid (Hkv, B), block NT.  KPT = 0: keys re-read from the scores (lists
// longer than NT * 16 units).
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_kernel(
    const float* __restrict__ scores, int max_units, int hkv, const int32_t* __restrict__ lens,
    int max_pages, int unit_tokens, int k, int n_head, int n_tail, int32_t* __restrict__ sel,
    int32_t* __restrict__ num_sel, int max_sel) {
  __shared__ TopkSmem<NT> sm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(lens[b], max_pages);
  const int n = (L + unit_tokens - 1) / unit_tokens;
  const int np = (L + kPage - 1) / kPage;
  const size_t list = (size_t)b * hkv + h;
  topk_list<NT, KPT, false>(scores ? scores + list * max_units : nullptr, n, np, unit_tokens / kPage,
                            k, n_head, n_tail, sel + list * max_sel, num_sel + list, max_sel, sm);
}

}  // namespace

hipError_t launch_topk(const float* scores, int max_units, const Shapes& s, const int32_t* lens,
                       int unit_tokens, int k, int n_head, int n_tail, int32_t* sel,
                       int32_t* num_sel, int max_sel, hipStream_t st) {
  if (max_units <= 1024 * 4)
    hipLaunchKernelGGL((topk_kernel<1024, 4>), dim3(s.Hkv, s.B), dim3(1024), 0, st, scores,
                       max_units, s.Hkv, lens, s.max_pages, unit_tokens, k, n_head, n_tail, sel,
                       num_sel, max_sel);
  else if (max_units <= 1024 * 16)
    hipLaunchKernelGGL((topk_kernel<1024, 16>), dim3(s.Hkv, s.B), dim3(1024), 0, st, scores,
                       max_units, s.Hkv, lens, s.max_pages, unit_tokens, k, n_head, n_tail, sel,
                       num_sel, max_sel);
  else
    hipLaunchKernelGGL((topk_kernel<1024, 0>), dim3(s.Hkv, s.B), dim3(1024), 0, st, scores,
                       max_units, s.Hkv, lens, s.max_pages, unit_tokens, k, n_head, n_tail, sel,
                       num_sel, max_sel);
  return hipGetLastError();
}

}  // namespace sa
