// sa_dev_topk.h - exact top-K of one (batch, kv-head) list inside one
// workgroup of NT threads (device code shared by the standalone top-K kernel
// and the fused decode-step kernel).
//
// Semantics ("SALS长序列推理优化", QSI top-k: exact, stable descending order;
// "Day 10·2 sparse top-k": lower index wins ties, the last block is always
// kept, nothing is padded below k; "Quest 完全拆解": the kept page numbers are
// the attention kernel's sparse-load indices): keep the n_head first and
// n_tail last units and the k best middle units by (score desc, index asc);
// emit the kept units' logical pages in ascending order.
//
// Method (no sort): scores become order-preserving uint32 keys (-0.0 folded
// into +0.0); the block min/max of the keys gives their common high-bit
// prefix, which is skipped; 8-bit radix-select passes (LDS histogram, one bin
// per thread, block scan from the largest digit) find the exact k-th largest
// key T and how many T-valued keys r are kept; with every thread owning a
// contiguous run of units, one block scan of (#keys > T, #keys == T) ranks
// each kept unit in index order.  A unit equal to T is kept iff fewer than r
// equal units precede it (the lower-index tie rule), and its rank is its
// output slot, so the list comes out ascending.
#pragma once

#include "sa_internal.h"

namespace sa {

// CAP: keys staged in LDS (one padding word per 32 keys against bank
// conflicts of the per-thread runs); longer lists re-read their scores.
template <int NT, int CAP>
struct TopkSmem {
  uint32_t keys[CAP + CAP / 32];
  uint32_t hist[256];
  uint32_t wa[NT / 64 + 1], wb[NT / 64 + 1];
  uint32_t bc[4];
  int last_kept;
};

__device__ __forceinline__ int key_slot(int u) { return u + (u >> 5); }

__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0.0 -> +0.0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of two counters over the NT threads of the block; returns
// the exclusive prefixes.  Two barriers.
template <int NT, int CAP>
__device__ __forceinline__ void block_exscan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                              TopkSmem<NT, CAP>& sm) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t va = a, vb = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t ua = __shfl_up(va, d, 64), ub = __shfl_up(vb, d, 64);
    if (lane >= d) { va += ua; vb += ub; }
  }
  if (lane == 63) { sm.wa[wave] = va; sm.wb[wave] = vb; }
  __syncthreads();
  uint32_t oa = 0, ob = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) { oa += sm.wa[w]; ob += sm.wb[w]; }
  }
  ea = va - a + oa;
  eb = vb - b + ob;
  __syncthreads();
}

// Selection of one list.  sc: the list's scores (unit 0 first); n units, np
// pages, upu pages per unit.  COH: scores are read and the page list is
// written with device-coherent accesses.  All NT threads call.
template <int NT, int CAP, bool COH = false>
__device__ void topk_list(const float* __restrict__ sc, int n, int np, int upu, int k, int n_head,
                          int n_tail, int32_t* __restrict__ out, int32_t* __restrict__ out_n,
                          int max_sel, TopkSmem<NT, CAP>& sm) {
  const int tid = threadIdx.x;
  if (n <= n_head + n_tail + k) {  // every unit is kept; no padding
    const int cnt = min(np, max_sel);
    for (int i = tid; i < max_sel; i += NT) st_x<COH>(out + i, i < cnt ? i : -1);
    if (tid == 0) st_x<COH>(out_n, cnt);
    return;
  }
  const int m = n - n_head - n_tail;  // competing middle units; m > k >= 0
  const float* msc = sc + n_head;
  const int run = (m + NT - 1) / NT;
  const int r0 = min(tid * run, m), r1 = min(r0 + run, m);
  const bool staged = m <= CAP;
  if (staged) {
    // all loads of a thread are issued before the first is used
    constexpr int PER = (CAP + NT - 1) / NT;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * NT;
      v[j] = u < m ? ld_x<COH>(msc + u) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = tid + j * NT;
      if (u < m) sm.keys[key_slot(u)] = order_key(v[j]);
    }
    __syncthreads();
  }
  // visit the thread's keys in index order
  auto for_keys = [&](auto&& f) {
    if (staged) {
      for (int j = 0; j < r1 - r0; ++j) f(j, sm.keys[key_slot(r0 + j)]);
    } else {
      for (int j = 0; j < r1 - r0; ++j) f(j, order_key(ld_x<COH>(msc + r0 + j)));
    }
  };

  if (tid == 0) sm.last_kept = n_tail > 0 ? 1 : 0;
  uint32_t T = 0xFFFFFFFFu, rem = 0;
  if (k > 0) {
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for_keys([&](int, uint32_t x) { kmin = min(kmin, x); kmax = max(kmax, x); });
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, 64));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) { sm.wa[wave] = kmin; sm.wb[wave] = kmax; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) { kmin = min(kmin, sm.wa[w]); kmax = max(kmax, sm.wb[w]); }
    __syncthreads();
    rem = (uint32_t)k;
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0u) {
      T = kmax;  // all keys equal: the k lowest indices are kept
    } else {
      int nb = 32 - __clz(diff);              // bits still undetermined
      uint64_t prefix = (uint64_t)kmax >> nb;  // the determined high bits
      while (nb > 0) {
        const int w = nb < 8 ? nb : 8;
        const int shift = nb - w;
        const uint32_t dmask = (1u << w) - 1u;
        for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
        __syncthreads();
        for_keys([&](int, uint32_t x) {
          if (((uint64_t)x >> nb) == prefix) atomicAdd(&sm.hist[(x >> shift) & dmask], 1u);
        });
        __syncthreads();
        // bins from the largest digit down: thread t takes bins 4t .. 4t+3 of the
        // descending order (one bin per thread for NT = 256)
        constexpr int BPT = (256 + NT - 1) / NT;
        uint32_t cnt[BPT], tot = 0;
#pragma unroll
        for (int jj = 0; jj < BPT; ++jj) {
          const int bin = (1 << w) - 1 - (tid * BPT + jj);
          cnt[jj] = bin >= 0 ? sm.hist[bin] : 0u;
          tot += cnt[jj];
        }
        uint32_t before, unused;
        block_exscan2<NT, CAP>(tot, 0u, before, unused, sm);
#pragma unroll
        for (int jj = 0; jj < BPT; ++jj) {
          const int bin = (1 << w) - 1 - (tid * BPT + jj);
          if (bin >= 0 && before < rem && rem <= before + cnt[jj]) {
            sm.bc[0] = (uint32_t)bin;
            sm.bc[1] = rem - before;
          }
          before += cnt[jj];
        }
        __syncthreads();
        prefix = (prefix << w) | sm.bc[0];
        rem = sm.bc[1];
        nb = shift;
      }
      T = (uint32_t)prefix;
    }
  }

  uint32_t gt = 0, eq = 0;
  if (k > 0) for_keys([&](int, uint32_t x) { gt += x > T; eq += x == T; });
  uint32_t gt_before, eq_before;
  block_exscan2<NT, CAP>(gt, eq, gt_before, eq_before, sm);

  const int last_pages = np - (n - 1) * upu;  // pages of the final (possibly partial) unit
  auto emit = [&](int rank, int u) {
    const int cntp = (u == n - 1) ? last_pages : upu;
    for (int i = 0; i < cntp; ++i) {
      const int pos = rank * upu + i;
      if (pos < max_sel) st_x<COH>(out + pos, u * upu + i);
    }
  };
  if (k > 0) {
    uint32_t kept_before = gt_before + min(eq_before, rem);
    uint32_t eq_seen = eq_before;
    for_keys([&](int j, uint32_t x) {
      bool keep = x > T;
      if (x == T) {
        keep = eq_seen < rem;
        ++eq_seen;
      }
      if (keep) {
        emit(n_head + (int)kept_before, n_head + r0 + j);
        ++kept_before;
        if (n_head + r0 + j == n - 1) sm.last_kept = 1;
      }
    });
  }
  for (int u = tid; u < n_head; u += NT) emit(u, u);
  for (int j = tid; j < n_tail; j += NT) emit(n_head + k + j, n - n_tail + j);
  __syncthreads();
  const int kept_units = n_head + k + n_tail;
  const int cnt = min(kept_units * upu - (sm.last_kept ? upu - last_pages : 0), max_sel);
  for (int i = cnt + tid; i < max_sel; i += NT) st_x<COH>(out + i, -1);
  if (tid == 0) st_x<COH>(out_n, cnt);
}

}  // namespace sa
