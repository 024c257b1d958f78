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
// -0.0 folded into +0.0).  The block min/max of the keys fixes their common
// high bits.  Radix-select passes over 8-bit digits of the undetermined bits
// then narrow a threshold prefix: LDS histogram by atomics, one barrier, and
// every wave scans all 256 bins itself (4 per lane, DPP prefix sum, ballot)
// so that all waves agree on the digit without a second barrier.  Three
// histograms rotate, each cleared two passes before its next use.  The passes
// stop once the threshold prefix is fully determined or once every key that
// carries it is kept (a few keys left at the threshold cost one more cheap
// pass, which beats ranking them).  One block scan of (#keys above, #keys at the threshold)
// then ranks every kept unit in index order: a unit at the threshold is kept
// iff fewer than r such units precede it (the lower-index tie rule), and its
// rank is its output slot, so the list comes out ascending without sorting.
//
// Lists longer than NT * KPT units use the same passes with the keys re-read
// from the scores (KPT = 0).  The core hands every kept unit with its output
// rank to a caller-supplied function, so a caller can write the list, or keep
// only the units of its own page range.
#pragma once

#include "sa_internal.h"

namespace sa {

constexpr int kTopkDigit = 8;
constexpr int kTopkBins = 1 << kTopkDigit;

// The KEYS hand-off's fallback when a key has not arrived in time: the
// caller's help object produces the missing keys itself.  mark(u) is called by
// every thread for each of its units still missing (u in [n_head, n - n_tail)),
// then, after a barrier, run() by all NT threads; run() must have stored every
// marked unit's key, device-coherently and completed, before it returns.
struct NoHelp {
  __device__ __forceinline__ void mark(int) const {}
  __device__ __forceinline__ void run() const {}
};

// How long a KEYS reader polls for keys still at 0 before it asks for help:
// s_memrealtime ticks (100 MHz), about 20 us, far above the usual spread of
// a few microseconds between the first and the last chunk of a list.
constexpr uint64_t kKeyWaitTicks = 2000;

template <int NT>
struct TopkSmem {
  alignas(16) uint32_t hist[3][kTopkBins];
  uint32_t wmin[NT / 64], wmax[NT / 64], wmiss[NT / 64];
  uint32_t wa[NT / 64], wb[NT / 64];
  int last_kept;
};

// Selection core of one list.  sc: the list's n unit scores.  Calls
// keep(rank, u) exactly once for every kept unit u (any thread may make a
// call).  With want_rank, rank is u's position among the kept units in
// ascending unit order; otherwise it is -1 and the ranking scan is skipped
// unless exact ties need it.  KPT > 0 requires n - n_head - n_tail <= NT * KPT.
// COH: the scores are read device-coherently.  KEYS (KPT > 0 only): sc holds
// order_key() words written by other workgroups, 0 while not yet written; such
// words are re-read for up to kKeyWaitTicks, and any still missing then are
// produced through help (so the call never depends on another workgroup
// being resident).  With k = 0 the keys are not needed and nothing is waited
// for.  All NT threads call; sm is free again on return once the caller has
// synchronised.
template <int NT, int KPT, bool COH, bool KEYS = false, typename Keep, typename Help = NoHelp>
__device__ __forceinline__ void topk_core(const float* __restrict__ sc, int n, int k, int n_head,
                                          int n_tail, TopkSmem<NT>& sm, Keep&& keep,
                                          bool want_rank = true, const Help& help = Help{}) {
  static_assert(!KEYS || KPT > 0, "key hand-off needs register-resident keys");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (n <= n_head + n_tail + k) {  // every unit is kept; no padding
    for (int u = tid; u < n; u += NT) keep(want_rank ? u : -1, u);
    return;
  }
  const int m = n - n_head - n_tail;  // competing middle units; m > k >= 0
  const float* msc = sc + n_head;
  // Scores (not KEYS) with KPT a multiple of 4: the runs are cut from the
  // absolute units 0 .. n - 1, so that a run starts on a multiple of 4 units
  // and is read with 16-byte loads; head and tail units inside a run are not
  // keys.  Otherwise the runs are cut from the middle units.
  constexpr bool kAbs = !KEYS && KPT > 0 && KPT % 4 == 0;
  const int run = kAbs ? (n + NT - 1) / NT : (m + NT - 1) / NT;
  const int r0 = kAbs ? min(tid * run, n) - n_head : min(tid * run, m);  // the run's first unit - n_head
  const int j_lo = kAbs ? max(0, -r0) : 0;                          // keys j_lo .. cnt_t - 1
  const int cnt_t = max(0, min(run, m - r0));

  // keys of the run: one round trip.  Loads are unconditional from clamped
  // in-range indices so that they are all in flight together; out-of-run
  // values are discarded afterwards.
  uint32_t key[KPT > 0 ? KPT : 1];
  const uint32_t* mk = reinterpret_cast<const uint32_t*>(sc) + n_head;  // KEYS: the order-key words
  bool missing = false;  // KEYS: a key of this thread's run has not arrived
  if constexpr (KEYS) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = ld_x<true>(mk + min(r0 + j, m - 1));
#pragma unroll
    for (int j = 0; j < KPT; ++j) missing |= j < cnt_t && key[j] == 0u;
    if (k == 0) missing = false;  // no competing unit is kept: the keys are not needed
    if (missing) {  // stores not yet landed: re-read those words, for a bounded time
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + kKeyWaitTicks;
      while (missing && __builtin_amdgcn_s_memrealtime() < t_end) {
        __builtin_amdgcn_s_sleep(1);
        missing = false;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          if (j < cnt_t && key[j] == 0u) {
            key[j] = ld_x<true>(mk + r0 + j);
            missing |= key[j] == 0u;
          }
        }
      }
    }
    // keys still missing are produced through help once the block knows of
    // them (at the barrier of the key bounds below)
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = j < cnt_t ? key[j] : 0u;
  } else if constexpr (KPT > 0) {
    float v[KPT];
    const float* rs = sc + (n_head + r0);  // kAbs: the run's first unit
    if (kAbs && !COH && run % 4 == 0 && n_head + r0 + run <= n &&
        (reinterpret_cast<uintptr_t>(rs) & 15u) == 0) {
#pragma unroll
      for (int j = 0; j < KPT; j += 4)
        if (j < run) *reinterpret_cast<float4*>(&v[j]) = *reinterpret_cast<const float4*>(rs + j);
    } else if (kAbs) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) v[j] = ld_x<COH>(sc + min(n_head + r0 + j, n - 1));
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) v[j] = ld_x<COH>(msc + min(r0 + j, m - 1));
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = (j >= j_lo && j < cnt_t) ? order_key(v[j]) : 0u;
  }
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (KPT > 0) return key[j];
    else return order_key(ld_x<COH>(msc + r0 + j));
  };
  auto for_keys = [&](auto&& f) {
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (j >= j_lo && j < cnt_t) f(j, key[j]);
    } else {
      for (int j = 0; j < cnt_t; ++j) f(j, key_at(j));
    }
  };

  for (int i = tid; i < 3 * kTopkBins; i += NT) (&sm.hist[0][0])[i] = 0u;

  // threshold: keys whose bits under mask dm equal tval ("at" keys, cbin of
  // them); rem of them are kept, every key above is kept
  uint32_t dm = 0xFFFFFFFFu, tval = 0xFFFFFFFFu, rem = 0, cbin = 0;
  if (k > 0) {
    // block min/max of the keys; with KEYS the same barrier tells every
    // thread whether any key of the list is still missing
    uint32_t kmin, kmax;
    auto bounds = [&]() -> bool {
      kmin = 0xFFFFFFFFu;
      kmax = 0u;
      for_keys([&](int, uint32_t x) { kmin = min(kmin, x); kmax = max(kmax, x); });
      kmin = wave_min_u32(kmin);
      kmax = wave_max_u32(kmax);
      const uint32_t miss = (KEYS && __ballot(missing ? 1 : 0) != 0ull) ? 1u : 0u;
      if (lane == 0) { sm.wmin[wave] = kmin; sm.wmax[wave] = kmax; sm.wmiss[wave] = miss; }
      __syncthreads();  // also orders the histogram clears before the first pass
      uint32_t any = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kmin = min(kmin, sm.wmin[w]);
        kmax = max(kmax, sm.wmax[w]);
        any |= sm.wmiss[w];
      }
      return any != 0u;
    };
    if (bounds()) {  // KEYS only: missing keys; their units are produced here
      if constexpr (KEYS) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (j < cnt_t && key[j] == 0u) help.mark(n_head + r0 + j);
        __syncthreads();
        help.run();
        __syncthreads();
        // every key is read again, so that none is held in registers while help runs
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = ld_x<true>(mk + min(r0 + j, m - 1));
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = j < cnt_t ? key[j] : 0u;
        missing = false;
        (void)bounds();
      }
    }
    rem = (uint32_t)k;
    const uint32_t diff = kmin ^ kmax;
    tval = kmax;
    cbin = (uint32_t)m;  // all keys are equal when diff == 0
    if (diff != 0u) {
      int nb = 32 - __clz(diff);  // low bits still undetermined
      dm = nb >= 32 ? 0u : 0xFFFFFFFFu << nb;
      tval = kmax & dm;
      for (int pass = 0;; ++pass) {
        const int w = nb < kTopkDigit ? nb : kTopkDigit;
        const int shift = nb - w;
        const int off = kTopkBins - (1 << w);  // bin of digit 0: the largest digit is bin 255
        const uint32_t dmask = (1u << w) - 1u;
        uint32_t* H = sm.hist[pass % 3];
        for_keys([&](int, uint32_t x) {
          if ((x & dm) == tval) atomicAdd(&H[off + (int)((x >> shift) & dmask)], 1u);
        });
        __syncthreads();
        {  // last read one pass ago, next counted into two passes ahead
          uint32_t* C = sm.hist[(pass + 2) % 3];
          for (int i = tid; i < kTopkBins; i += NT) C[i] = 0u;
        }
        // every wave: lane l holds bins 255-4l .. 252-4l, largest first
        const uint4 hv = *reinterpret_cast<const uint4*>(&H[kTopkBins - 4 - 4 * lane]);
        const uint32_t c4[4] = {hv.w, hv.z, hv.y, hv.x};
        const uint32_t tot = hv.x + hv.y + hv.z + hv.w;
        const uint32_t incl = wave_incl_scan_u32(tot);
        uint32_t before = incl - tot;
        const uint64_t hit = __ballot(before < rem && rem <= incl);  // exactly one lane
        const int src = __ffsll((unsigned long long)hit) - 1;
        int bin = 0;
        uint32_t nrem = 0;
        cbin = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (before < rem && rem <= before + c4[jj]) {
            bin = kTopkBins - 1 - 4 * lane - jj;
            cbin = c4[jj];
            nrem = rem - before;
          }
          before += c4[jj];
        }
        bin = __builtin_amdgcn_readlane(bin, src);
        cbin = (uint32_t)__builtin_amdgcn_readlane((int)cbin, src);
        rem = (uint32_t)__builtin_amdgcn_readlane((int)nrem, src);
        tval |= (uint32_t)(bin - off) << shift;
        dm |= dmask << shift;
        nb = shift;
        if (nb == 0 || cbin == rem) break;  // fully determined, or the whole bin is kept
      }
    }
  }
  // At keys are all kept (cbin == rem), or else (exact ties) the first rem in
  // unit order, which needs a block scan of the at keys; the output ranks
  // need a block scan of the kept keys.
  const bool tie_scan = k > 0 && cbin != rem;
  const bool scan = k > 0 && (tie_scan || want_rank);
  uint32_t kept_before = 0, eq_seen = 0;
  if (scan) {
    uint32_t gt = 0, eq = 0;
    for_keys([&](int j, uint32_t x) {
      const uint32_t xm = x & dm;
      gt += xm > tval;
      eq += xm == tval;
    });
    const uint32_t ga = wave_incl_scan_u32(gt), ea = wave_incl_scan_u32(eq);
    if (lane == 63) { sm.wa[wave] = ga; sm.wb[wave] = ea; }
    __syncthreads();
    uint32_t gt_before = ga - gt, eq_before = ea - eq;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2)
      if (w2 < wave) { gt_before += sm.wa[w2]; eq_before += sm.wb[w2]; }
    kept_before = gt_before + (tie_scan ? min(eq_before, rem) : eq_before);
    eq_seen = eq_before;
  }
  if (k > 0) {
    for_keys([&](int j, uint32_t x) {
      const int u = n_head + r0 + j;
      const uint32_t xm = x & dm;
      bool kp = xm > tval;
      if (xm == tval) {
        if (tie_scan) {
          kp = eq_seen < rem;
          ++eq_seen;
        } else {
          kp = true;
        }
      }
      if (kp) {
        keep(scan && want_rank ? n_head + (int)kept_before : -1, u);
        ++kept_before;
      }
    });
  }
  // forced units: c < n_head is head unit c (rank c); else tail unit n - n_tail + j (rank n_head + k + j)
  for (int c = tid; c < n_head + n_tail; c += NT) {
    const bool head = c < n_head;
    const int rank = head ? c : n_head + k + (c - n_head);
    keep(want_rank ? rank : -1, head ? c : n - n_tail + (c - n_head));
  }
}

// Selection of one list written as a page list.  sc: the list's scores (unit 0
// first, n units, np pages, upu pages per unit).  out: the kept units' pages
// in ascending order, then -1 up to max_sel; out_n: their count.
template <int NT, int KPT, bool COH>
__device__ __forceinline__ void topk_list(const float* __restrict__ sc, int n, int np, int upu, int k,
                                          int n_head, int n_tail, int32_t* __restrict__ out,
                                          int32_t* __restrict__ out_n, int max_sel,
                                          TopkSmem<NT>& sm) {
  const int tid = threadIdx.x;
  const bool all = n <= n_head + n_tail + k;
  // written before any barrier of the core, which orders it before the kept units' writes
  if (tid == 0) sm.last_kept = (all || n_tail > 0) ? 1 : 0;
  const int last_pages = np - (n - 1) * upu;  // pages of the final (possibly partial) unit
  topk_core<NT, KPT, COH>(sc, n, k, n_head, n_tail, sm, [&](int rank, int u) {
    const int cntp = (u == n - 1) ? last_pages : upu;
    for (int i = 0; i < cntp; ++i) {
      const int pos = rank * upu + i;
      if (pos < max_sel) st_x<COH>(out + pos, u * upu + i);
    }
    if (u == n - 1 && !all) sm.last_kept = 1;
  });
  if (!all && upu > 1 && n_tail == 0) __syncthreads();  // only then can the final unit be dropped
  const int kept_units = all ? n : n_head + k + n_tail;
  const int cnt = n <= 0 ? 0 : min(kept_units * upu - (sm.last_kept ? upu - last_pages : 0), max_sel);
  for (int i = cnt + tid; i < max_sel; i += NT) st_x<COH>(out + i, -1);
  if (tid == 0) st_x<COH>(out_n, cnt);
}

}  // namespace sa
