// sa_topk.hip - exact top-K unit selection (step 2 of the decode step).
//
// Semantics ("SALS长序列推理优化", QSI top-k: exact, stable descending order;
// "Day 10·2 sparse top-k" page: the lower block index wins ties, the last
// block is always kept, nothing is padded below k; "Quest 完全拆解": the top-K
// page numbers become the attention kernel's sparse-load indices):
//   per (b, kv-head) keep the n_head first and n_tail last units, plus the
//   k best middle units ordered by (score desc, index asc), and emit the kept
//   units' logical pages in ascending order.
//
// Design (one 1024-thread workgroup per list, no sort):
//   1. scores -> order-preserving uint32 keys (-0.0 folded into +0.0);
//   2. block min/max of the keys gives their common high-bit prefix, which is
//      skipped; the remaining bits are resolved by 8-bit radix-select passes
//      (LDS histogram, one wave scans the 256 bins from the top) until the
//      exact k-th largest key T and the number r of T-valued keys to keep are
//      known;
//   3. with each thread owning a contiguous run of units, one block-wide
//      exclusive scan of (#keys > T, #keys == T) gives every kept unit its
//      rank in index order: a unit equal to T is kept iff fewer than r equal
//      units precede it, which is exactly the lower-index tie rule.  The ranks
//      are the output positions, so the list comes out ascending.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kKeysPerThread = 16;  // register-resident keys: lists of up to 16384 middle units

__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0.0 -> +0.0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Visit the keys of a thread's run; register-resident runs are fully unrolled.
template <bool REGS, typename F>
__device__ __forceinline__ void for_keys(int r0, int r1, F&& f) {
  if constexpr (REGS) {
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j)
      if (r0 + j < r1) f(j);
  } else {
    for (int j = 0; j < r1 - r0; ++j) f(j);
  }
}

// Exclusive block scan of two counters; returns the totals through refs.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                            uint32_t& ta, uint32_t& tb, uint32_t* s_a,
                                            uint32_t* s_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t va = a, vb = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t ua = __shfl_up(va, d, 64), ub = __shfl_up(vb, d, 64);
    if (lane >= d) { va += ua; vb += ub; }
  }
  if (lane == 63) { s_a[wave] = va; s_b[wave] = vb; }
  __syncthreads();
  if (wave == 0) {
    uint32_t wa = lane < kTopkWaves ? s_a[lane] : 0u, wb = lane < kTopkWaves ? s_b[lane] : 0u;
    uint32_t xa = wa, xb = wb;
#pragma unroll
    for (int d = 1; d < kTopkWaves; d <<= 1) {
      const uint32_t ua = __shfl_up(xa, d, 64), ub = __shfl_up(xb, d, 64);
      if (lane >= d) { xa += ua; xb += ub; }
    }
    if (lane < kTopkWaves) { s_a[kTopkWaves + lane] = xa - wa; s_b[kTopkWaves + lane] = xb - wb; }
    if (lane == kTopkWaves - 1) { s_a[2 * kTopkWaves] = xa; s_b[2 * kTopkWaves] = xb; }
  }
  __syncthreads();
  ea = va - a + s_a[kTopkWaves + wave];
  eb = vb - b + s_b[kTopkWaves + wave];
  ta = s_a[2 * kTopkWaves];
  tb = s_b[2 * kTopkWaves];
}

// grid (Hkv, B), block 1024.  REGS: keys of the thread's run held in registers
// (run length <= kKeysPerThread); otherwise re-read from the scores each pass.
template <bool REGS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, int max_units, int hkv, const int32_t* __restrict__ lens,
    int max_pages, int unit_tokens, int k, int n_head, int n_tail, int32_t* __restrict__ sel,
    int32_t* __restrict__ num_sel, int max_sel) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_a[2 * kTopkWaves + 1], s_b[2 * kTopkWaves + 1];
  __shared__ uint32_t s_bc[4];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = clamp_len(lens[b], max_pages);
  const int n = (L + unit_tokens - 1) / unit_tokens;
  const int np = (L + kPage - 1) / kPage;
  const int upu = unit_tokens / kPage;
  int32_t* out = sel + ((size_t)b * hkv + h) * max_sel;
  int32_t* out_n = num_sel + (size_t)b * hkv + h;

  if (n <= n_head + n_tail + k) {  // every unit is kept; no padding [Day 10·2]
    const int cnt = min(np, max_sel);
    for (int i = tid; i < max_sel; i += kTopkThreads) out[i] = i < cnt ? i : -1;
    if (tid == 0) *out_n = cnt;
    return;
  }

  // the final unit is kept iff it is a tail unit or a kept middle unit
  __shared__ int s_last_kept;
  if (tid == 0) s_last_kept = n_tail > 0 ? 1 : 0;  // ordered by the barriers below

  const int m = n - n_head - n_tail;  // middle units compete; m > k >= 0
  const float* sc = scores + ((size_t)b * hkv + h) * max_units + n_head;
  const int run = (m + kTopkThreads - 1) / kTopkThreads;
  const int r0 = min(tid * run, m), r1 = min(r0 + run, m);

  uint32_t key[REGS ? kKeysPerThread : 1];
  if constexpr (REGS) {
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) key[j] = (r0 + j < r1) ? order_key(sc[r0 + j]) : 0u;
  } else {
    key[0] = 0u;
  }
  auto get_key = [&](int j) -> uint32_t {
    if constexpr (REGS) return key[j];
    else return order_key(sc[r0 + j]);
  };

  uint32_t T = 0xFFFFFFFFu;  // threshold key
  uint32_t rem = 0;          // keys equal to T that are kept
  if (k > 0) {
    // common high-bit prefix of all middle keys
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for_keys<REGS>(r0, r1, [&](int j) {
      const uint32_t x = get_key(j);
      kmin = min(kmin, x);
      kmax = max(kmax, x);
    });
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, 64));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
    }
    if (lane == 0) { s_a[wave] = kmin; s_b[wave] = kmax; }
    __syncthreads();
    if (tid == 0) {
      uint32_t a = s_a[0], c = s_b[0];
      for (int w = 1; w < kTopkWaves; ++w) { a = min(a, s_a[w]); c = max(c, s_b[w]); }
      s_bc[0] = a;
      s_bc[1] = c;
    }
    __syncthreads();
    kmin = s_bc[0];
    kmax = s_bc[1];
    __syncthreads();
    const uint32_t diff = kmin ^ kmax;
    rem = (uint32_t)k;
    if (diff == 0u) {
      T = kmax;  // all keys equal: keep the k lowest indices
    } else {
      int nb = 32 - __clz(diff);  // undetermined low bits
      uint64_t prefix = (uint64_t)kmax >> nb;
      while (nb > 0) {
        const int w = nb < 8 ? nb : 8;
        const int shift = nb - w;
        const uint32_t dmask = (1u << w) - 1u;
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        for_keys<REGS>(r0, r1, [&](int j) {
          const uint32_t x = get_key(j);
          if (((uint64_t)x >> nb) == prefix) atomicAdd(&hist[(x >> shift) & dmask], 1u);
        });
        __syncthreads();
        if (wave == 0) {
          // lane l scans bins (nbins-1-4l) down to (nbins-4-4l): the largest digits first
          const int nbins = 1 << w;
          uint32_t cnt[4], tot = 0;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int bin = nbins - 1 - (4 * lane + jj);
            cnt[jj] = bin >= 0 ? hist[bin] : 0u;
            tot += cnt[jj];
          }
          uint32_t inc = tot;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            const uint32_t u = __shfl_up(inc, d, 64);
            if (lane >= d) inc += u;
          }
          uint32_t before = inc - tot;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int bin = nbins - 1 - (4 * lane + jj);
            if (bin >= 0 && before < rem && rem <= before + cnt[jj]) {
              s_bc[2] = (uint32_t)bin;
              s_bc[3] = rem - before;
            }
            before += cnt[jj];
          }
        }
        __syncthreads();
        prefix = (prefix << w) | s_bc[2];
        rem = s_bc[3];
        nb = shift;
        __syncthreads();
      }
      T = (uint32_t)prefix;
    }
  }

  // rank every kept middle unit in index order
  uint32_t gt = 0, eq = 0;
  if (k > 0) {
    for_keys<REGS>(r0, r1, [&](int j) {
      const uint32_t x = get_key(j);
      gt += x > T;
      eq += x == T;
    });
  }
  uint32_t gt_before, eq_before, gt_tot, eq_tot;
  block_scan2(gt, eq, gt_before, eq_before, gt_tot, eq_tot, s_a, s_b);

  const int last_pages = np - (n - 1) * upu;  // pages of the final (possibly partial) unit
  auto emit = [&](int rank, int u) {
    const int p0 = u * upu;
    const int cntp = (u == n - 1) ? last_pages : upu;
    for (int i = 0; i < cntp; ++i) {
      const int pos = rank * upu + i;
      if (pos < max_sel) out[pos] = p0 + i;
    }
  };
  if (k > 0) {
    uint32_t kept_before = gt_before + min(eq_before, rem);
    uint32_t eq_seen = eq_before;
    for_keys<REGS>(r0, r1, [&](int j) {
      const uint32_t x = get_key(j);
      bool keep = x > T;
      if (x == T) {
        keep = eq_seen < rem;
        ++eq_seen;
      }
      if (keep) {
        emit(n_head + (int)kept_before, n_head + r0 + j);
        ++kept_before;
        if (n_head + r0 + j == n - 1) s_last_kept = 1;
      }
    });
  }
  for (int u = tid; u < n_head; u += kTopkThreads) emit(u, u);
  for (int j = tid; j < n_tail; j += kTopkThreads) emit(n_head + k + j, n - n_tail + j);

  __syncthreads();
  const int kept_units = n_head + k + n_tail;
  const int cnt = min(kept_units * upu - (s_last_kept ? upu - last_pages : 0), max_sel);
  for (int i = cnt + tid; i < max_sel; i += kTopkThreads) out[i] = -1;
  if (tid == 0) *out_n = cnt;
}

}  // namespace

hipError_t launch_topk(const float* scores, int max_units, const Shapes& s, const int32_t* lens,
                       int unit_tokens, int k, int n_head, int n_tail, int32_t* sel,
                       int32_t* num_sel, int max_sel, hipStream_t st) {
  dim3 grid(s.Hkv, s.B);
  const int max_mid = max_units;  // upper bound of any list's middle-unit count
  if (max_mid <= kTopkThreads * kKeysPerThread)
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(kTopkThreads), 0, st, scores, max_units,
                       s.Hkv, lens, s.max_pages, unit_tokens, k, n_head, n_tail, sel, num_sel,
                       max_sel);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(kTopkThreads), 0, st, scores, max_units,
                       s.Hkv, lens, s.max_pages, unit_tokens, k, n_head, n_tail, sel, num_sel,
                       max_sel);
  return hipGetLastError();
}

}  // namespace sa
