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
// Method (no sort): every thread owns a contiguous run of middle units and
// keeps their order-preserving uint32 keys in registers (scores -> keys with
// -0.0 folded into +0.0).  The block min/max of the keys gives their common
// high-bit prefix, which is skipped; radix-select passes over 12-bit digits
// (LDS histograms used alternately, 16 bins per thread scanned from the
// largest digit) find the exact k-th largest key T and how many T-valued keys
// r are kept -- two passes for score sets that share sign and exponent.  One
// block scan of (#keys > T, #keys == T) then ranks every kept unit in index
// order: a unit equal to T is kept iff fewer than r equal units precede it
// (the lower-index tie rule), and its rank is its output slot, so the list
// comes out ascending without sorting.
//
// Lists longer than NT * KPT units use the same passes with the keys re-read
// from the scores (KPT = 0).
#pragma once

#include "sa_internal.h"

namespace sa {

constexpr int kTopkDigit = 12;
constexpr int kTopkBins = 1 << kTopkDigit;

template <int NT>
struct TopkSmem {
  uint32_t hist[2][kTopkBins];
  uint32_t wmin[NT / 64], wmax[NT / 64];
  uint32_t wsum[2][NT / 64];
  uint32_t bc[2][2];
  uint32_t wa[NT / 64], wb[NT / 64];
  int last_kept;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0.0 -> +0.0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A kept page as the attention tasks read it: (physical page << 4) | (valid tokens - 1),
// or -1 when the page-table entry is out of range.
__device__ __forceinline__ int32_t resolved_page(int pp, int nv, int num_pages) {
  return (pp >= 0 && pp < num_pages) ? ((pp << 4) | (nv - 1)) : -1;
}

// Selection of one list.  sc: the list's scores (unit 0 first, n units, np
// pages, upu pages per unit).  KPT > 0 requires n - n_head - n_tail <= NT * KPT.
// COH: scores are read and outputs written device-coherently.  rout (optional,
// upu == 1 only): the kept pages resolved through pt_row as resolved_page().
// All NT threads call.
template <int NT, int KPT, bool COH>
__device__ __forceinline__ void topk_list(const float* __restrict__ sc, int n, int np, int upu, int k, int n_head,
                          int n_tail, int32_t* __restrict__ out, int32_t* __restrict__ out_n,
                          int max_sel, TopkSmem<NT>& sm, const int32_t* __restrict__ pt_row = nullptr,
                          int L = 0, int num_pages = 0, int32_t* __restrict__ rout = nullptr) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto resolve = [&](int p) -> int32_t {
    return resolved_page(pt_row[p], min(kPage, L - p * kPage), num_pages);
  };

  if (n <= n_head + n_tail + k) {  // every unit is kept; no padding
    const int cnt = min(np, max_sel);
    for (int i = tid; i < max_sel; i += NT) {
      st_x<COH>(out + i, i < cnt ? i : -1);
      if (rout) st_x<COH>(rout + i, i < cnt ? resolve(i) : -1);
    }
    if (tid == 0) st_x<COH>(out_n, cnt);
    return;
  }
  const int m = n - n_head - n_tail;  // competing middle units; m > k >= 0
  const float* msc = sc + n_head;
  const int run = (m + NT - 1) / NT;
  const int r0 = min(tid * run, m);
  const int cnt_t = min(run, m - r0);

  // keys (and, when resolving, page-table entries) of the run: one round trip.
  // Loads are unconditional from clamped in-range indices so that they are all
  // in flight together; out-of-run values are discarded afterwards.
  uint32_t key[KPT > 0 ? KPT : 1];
  int32_t rp[KPT > 0 ? KPT : 1];
  if constexpr (KPT > 0) {
    float v[KPT];
    int32_t pv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int u = min(r0 + j, m - 1);
      v[j] = ld_x<COH>(msc + u);
      if (rout) pv[j] = pt_row[n_head + u];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int u = min(r0 + j, m - 1);
      key[j] = j < cnt_t ? order_key(v[j]) : 0u;
      rp[j] = (rout && j < cnt_t) ? resolved_page(pv[j], min(kPage, L - (n_head + u) * kPage), num_pages) : -1;
    }
  }
  // forced units' resolved pages, fetched now as well
  int32_t forced_rp = -1;
  if (rout) {
    const int c = min(tid, n_head + n_tail - 1);
    const int u = c < 0 ? 0 : (c < n_head ? c : n - n_tail + (c - n_head));
    const int32_t pv = pt_row[u];
    if (tid < n_head + n_tail) forced_rp = resolved_page(pv, min(kPage, L - u * kPage), num_pages);
  }
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (KPT > 0) return key[j];
    else return order_key(ld_x<COH>(msc + r0 + j));
  };
  auto for_keys = [&](auto&& f) {
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (j < cnt_t) f(j, key[j]);
    } else {
      for (int j = 0; j < cnt_t; ++j) f(j, key_at(j));
    }
  };

  {
    uint4* h4 = reinterpret_cast<uint4*>(&sm.hist[0][0]);
    for (int i = tid; i < 2 * kTopkBins / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
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
    if (lane == 0) { sm.wmin[wave] = kmin; sm.wmax[wave] = kmax; }
    __syncthreads();  // also orders the histogram clears before the first pass
#pragma unroll
    for (int w = 0; w < NW; ++w) { kmin = min(kmin, sm.wmin[w]); kmax = max(kmax, sm.wmax[w]); }
    rem = (uint32_t)k;
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0u) {
      T = kmax;  // all keys equal: the k lowest indices are kept
    } else {
      int nb = 32 - __clz(diff);               // bits still undetermined
      uint64_t prefix = (uint64_t)kmax >> nb;  // the determined high bits
      for (int pass = 0; nb > 0; ++pass) {
        const int w = nb < kTopkDigit ? nb : kTopkDigit;
        const int shift = nb - w;
        const int nbins = 1 << w;
        uint32_t* H = sm.hist[pass & 1];
        for_keys([&](int, uint32_t x) {
          if (((uint64_t)x >> nb) == prefix) atomicAdd(&H[(x >> shift) & (uint32_t)(nbins - 1)], 1u);
        });
        __syncthreads();
        {  // clear the other histogram for the next pass (its last reads preceded this pass)
          uint4* o4 = reinterpret_cast<uint4*>(&sm.hist[(pass + 1) & 1][0]);
          for (int i = tid; i < kTopkBins / 4; i += NT) o4[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        // thread t scans bins nbins-1-16t down to nbins-16-16t (largest digits first)
        constexpr int BPT = kTopkBins / NT;
        uint32_t tot = 0;
#pragma unroll
        for (int jj = 0; jj < BPT; ++jj) {
          const int bin = nbins - 1 - (BPT * tid + jj);
          tot += bin >= 0 ? H[bin] : 0u;
        }
        uint32_t incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t u = __shfl_up(incl, d, 64);
          if (lane >= d) incl += u;
        }
        if (lane == 63) sm.wsum[pass & 1][wave] = incl;
        __syncthreads();
        uint32_t before = incl - tot;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2)
          if (w2 < wave) before += sm.wsum[pass & 1][w2];
        if (before < rem && rem <= before + tot) {  // the k-th key's digit is in this thread's bins
          for (int jj = 0; jj < BPT; ++jj) {
            const int bin = nbins - 1 - (BPT * tid + jj);
            const uint32_t cj = bin >= 0 ? H[bin] : 0u;
            if (before < rem && rem <= before + cj) {
              sm.bc[pass & 1][0] = (uint32_t)bin;
              sm.bc[pass & 1][1] = rem - before;
            }
            before += cj;
          }
        }
        __syncthreads();
        prefix = (prefix << w) | sm.bc[pass & 1][0];
        rem = sm.bc[pass & 1][1];
        nb = shift;
      }
      T = (uint32_t)prefix;
    }
  }

  // rank the kept middle units in index order: one block scan of (#> T, #== T)
  uint32_t gt = 0, eq = 0;
  if (k > 0) for_keys([&](int, uint32_t x) { gt += x > T; eq += x == T; });
  uint32_t ga = gt, ea = eq;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t ug = __shfl_up(ga, d, 64), ue = __shfl_up(ea, d, 64);
    if (lane >= d) { ga += ug; ea += ue; }
  }
  if (lane == 63) { sm.wa[wave] = ga; sm.wb[wave] = ea; }
  __syncthreads();
  uint32_t gt_before = ga - gt, eq_before = ea - eq;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2)
    if (w2 < wave) { gt_before += sm.wa[w2]; eq_before += sm.wb[w2]; }

  const int last_pages = np - (n - 1) * upu;  // pages of the final (possibly partial) unit
  auto emit = [&](int rank, int u, int32_t r) {
    const int cntp = (u == n - 1) ? last_pages : upu;
    for (int i = 0; i < cntp; ++i) {
      const int pos = rank * upu + i;
      if (pos < max_sel) {
        st_x<COH>(out + pos, u * upu + i);
        if (rout) st_x<COH>(rout + pos, r);
      }
    }
  };
  if (k > 0) {
    uint32_t kept_before = gt_before + min(eq_before, rem);
    uint32_t eq_seen = eq_before;
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if (j < cnt_t) {
          const uint32_t x = key[j];
          bool keep = x > T;
          if (x == T) {
            keep = eq_seen < rem;
            ++eq_seen;
          }
          if (keep) {
            emit(n_head + (int)kept_before, n_head + r0 + j, rp[j]);
            ++kept_before;
            if (n_head + r0 + j == n - 1) sm.last_kept = 1;
          }
        }
      }
    } else {
      for (int j = 0; j < cnt_t; ++j) {
        const uint32_t x = key_at(j);
        bool keep = x > T;
        if (x == T) {
          keep = eq_seen < rem;
          ++eq_seen;
        }
        if (keep) {
          const int u = n_head + r0 + j;
          emit(n_head + (int)kept_before, u, rout ? resolve(u) : -1);
          ++kept_before;
          if (u == n - 1) sm.last_kept = 1;
        }
      }
    }
  }
  // forced units: c < n_head is head unit c (rank c); else tail unit n - n_tail + j (rank n_head + k + j)
  for (int c = tid; c < n_head + n_tail; c += NT) {
    const bool head = c < n_head;
    const int u = head ? c : n - n_tail + (c - n_head);
    const int rank = head ? c : n_head + k + (c - n_head);
    emit(rank, u, c == tid ? forced_rp : (rout ? resolve(u) : -1));
  }
  if (upu > 1 && n_tail == 0) __syncthreads();  // only then can the final unit be dropped
  const int kept_units = n_head + k + n_tail;
  const int cnt = min(kept_units * upu - (sm.last_kept ? upu - last_pages : 0), max_sel);
  for (int i = cnt + tid; i < max_sel; i += NT) {
    st_x<COH>(out + i, -1);
    if (rout) st_x<COH>(rout + i, -1);
  }
  if (tid == 0) st_x<COH>(out_n, cnt);
}

}  // namespace sa
