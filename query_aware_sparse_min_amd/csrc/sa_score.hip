// sa_score.hip - page / block scorers (step 1 of the decode step).
//
//  * Quest criticality estimation ("Quest 完全拆解" explainer, upper bound
//    from min/max metadata; GQA section): score = max over the group's query
//    heads of sum_i max(q_i m_i, q_i M_i).  The sum is evaluated in its
//    equivalent linear form q+ . M + q- . m (q+ = max(q, 0), q- = min(q, 0)):
//    a lane owns 8 dimensions of either the M row or the m row of a
//    (page, kv-head) unit, so one 64-lane load covers two units with
//    coalesced 256-byte rows, and a 32-lane tree reduction finishes each sum.
//  * SALS block scorer ("SALS长序列推理优化", QSI steps 1-3): index query =
//    group mean of q projected by P; per token s_t = scale_t * qt . c_t from
//    the int4 codes; per block a log-sum-exp of tau * s_t, kept as an online
//    (max, sum) pair in base 2 and merged across the lanes of a kv-head.
#include "sa_dev_score.h"

namespace sa {
namespace {

constexpr int kScoreIT = 2;                        // load pairs per lane
constexpr int kScorePagesPerWG = 16 * kScoreIT;     // 32 pages per workgroup

// grid (ceil(max_pages / 32), Hkv, B), block 256.  PH: one row of scores per
// query head ([B, Hq, max_pages]) instead of one per group.
template <int KT, int QT, int G, bool PH>
__global__ __launch_bounds__(256) void quest_score_kernel(
    const void* __restrict__ q, const void* __restrict__ meta, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    float* __restrict__ scores) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(lens[b], max_pages);
  const int n = (L + kPage - 1) / kPage;
  const int p0 = blockIdx.x * kScorePagesPerWG;
  if (p0 >= n) return;
  const size_t row0 = PH ? ((size_t)b * hkv + h) * G : (size_t)b * hkv + h;
  quest_score_range<KT, QT, G, kScoreIT, false, 4, false, PH>(
      q, meta, num_pages, hkv, b, h, pt + (size_t)b * max_pages, p0, min(p0 + kScorePagesPerWG, n),
      lens + b, max_pages, scores + row0 * max_pages, nullptr, max_pages);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaTilesPerWave = 2;                               // 16-page tiles in flight per wave
constexpr int kMfmaPagesPerWG = 4 * kMfmaTilesPerWave * 16;        // 128 pages per workgroup

// Quest scores of G (4..16) bf16 query heads over bf16 metadata on the matrix
// cores: the bound of head g on a page is the dot product of [q_g+ | q_g-]
// (256 values) with the page's [M | m] row pair (the 512 contiguous bytes of
// its metadata), so a 16-page tile is the 16 x 16 product of [q+ | q-] (heads
// as rows, G of 16 used) with the pages' rows as columns: eight
// v_mfma_f32_16x16x32_bf16 over the 256-deep sum.  Lane l supplies, for MFMA
// kk, elements 32 kk + 8 (l / 16) .. + 7 of head l % 16 (A) and of page l % 16
// of the tile (B: one 16-byte load), so each lane loads its page's 128 bytes
// as eight 16-byte pieces.  The result tile holds heads 4 (l / 16) + i of page
// l % 16 in lane l; the group score is their max over the G heads (PH: each
// head's own row of scores instead).
// grid (ceil(max_pages / 128), Hkv, B), block 256.
template <int G, bool PH>
__global__ __launch_bounds__(256) void quest_score_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    float* __restrict__ scores) {
  static_assert(G >= 4 && G <= 16, "heads fill the MFMA rows");
  const int h = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(lens[b], max_pages);
  const int n_valid = (L + kPage - 1) / kPage;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int pw0 = blockIdx.x * kMfmaPagesPerWG + wave * kMfmaTilesPerWave * 16;
  if (pw0 >= n_valid) return;
  const int32_t* pt_row = pt + (size_t)b * max_pages;

  // page-table entries and metadata of this wave's tiles: every load in flight at once
  int pg[kMfmaTilesPerWave], pp[kMfmaTilesPerWave];
#pragma unroll
  for (int t = 0; t < kMfmaTilesPerWave; ++t) {
    pg[t] = pw0 + 16 * t + col;
    pp[t] = pt_row[min(pg[t], n_valid - 1)];
  }
  uint4 mw[kMfmaTilesPerWave][8];
#pragma unroll
  for (int t = 0; t < kMfmaTilesPerWave; ++t) {
    const int ppl = (pp[t] >= 0 && pp[t] < num_pages) ? pp[t] : 0;
    const uint4* row = reinterpret_cast<const uint4*>(meta + ((size_t)h * num_pages + ppl) * 2 * kHeadDim);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) mw[t][kk] = row[4 * kk + kg];
  }
  // A: [q+ | q-] of head col (zero beyond G): k < 128 takes q+ of dim k, k >= 128 q- of dim k - 128
  uint4 aw[8] = {};
  if (col < G) {
    const uint4* qr = reinterpret_cast<const uint4*>(q + ((size_t)b * hkv * G + (size_t)h * G + col) * kHeadDim);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 w = qr[(4 * kk + kg) & 15];
      const bool neg_half = kk >= 4;  // the m row pairs with q-
      uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t neg = (x[e] & 0x8000u ? 0x0000FFFFu : 0u) | (x[e] & 0x80000000u ? 0xFFFF0000u : 0u);
        x[e] &= neg_half ? neg : ~neg;
      }
      aw[kk] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  }
  float* sc_row = scores + ((size_t)b * hkv + h) * max_pages;
#pragma unroll
  for (int t = 0; t < kMfmaTilesPerWave; ++t) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw[kk]),
                                                   __builtin_bit_cast(bf16x8_t, mw[t][kk]), acc, 0, 0, 0);
    const bool ok = pg[t] < n_valid && pp[t] >= 0 && pp[t] < num_pages;
    if constexpr (PH) {
      float* head_rows = scores + ((size_t)b * hkv + h) * G * max_pages;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * kg + i < G && pg[t] < n_valid)
          head_rows[(size_t)(4 * kg + i) * max_pages + pg[t]] = ok ? acc[i] : -INFINITY;
      continue;
    }
    float best = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * kg + i < G) best = fmaxf(best, acc[i]);
    best = pair32_max(pair16_max(best));
    if (kg == 0 && pg[t] < n_valid) sc_row[pg[t]] = ok ? best : -INFINITY;
  }
}

constexpr int kSalsUnitsPerWG = 8;  // blocks scored per workgroup, two per wave
constexpr int kQbarStride = kHeadDim + 4;  // padded rows: the MFMA reads 16 rows at one column
constexpr int kQDigits = 7;         // balanced base-16 digits of the fixed-point index query
constexpr int kQLoDigits = 4;       // digits summed into the low int32 partial
constexpr int kQFracBits = 26;      // |Q| <= 2^26 (seven balanced digits reach 1.25e8)
__host__ __device__ constexpr size_t sals_smem_bytes(int hkv) {
  return sizeof(float) * ((size_t)kHeadDim * kRank + (size_t)hkv * kQbarStride) +
         sizeof(uint32_t) * (size_t)hkv * (2 * kQDigits + 1);
}
constexpr int kSalsHeads = 8;       // kv-heads of one pass over a block's tokens

// Merge of two base-2 (max, sum) pairs; symmetric, so both partners of an
// exchange end with bit-identical values.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.0f : s * exp2f(m - mm);
  const float c = m2 == -INFINITY ? 0.0f : s2 * exp2f(m2 - mm);
  s = a + c;
  m = mm;
}

// grid (ceil(max_units / kSalsUnitsPerWG), B), block 256.  The workgroup first
// stages the batch row of q and the projection P in LDS (vector loads, one
// memory round trip), forms every kv-head's group-mean query and projects it,
// qt = qbar P, on the matrix cores (fp32 v_mfma_f32_16x16x4f32, 16 kv-heads
// per tile).  Each kv-head's qt becomes integers Q_j = rint(qt_j 2^(26-e)),
// 2^(e-1) <= max |qt_j| < 2^e, written as seven balanced base-16 digits packed
// as signed nibbles; a token's dot product with its sixteen int4 codes is then
// exact integer work (fourteen v_dot8_i32_i4, Horner over the high three and
// the low four digits into two int32 sums, so neither can overflow), joined
// by one fp32 fma (the only rounding) and scaled by 2^(e-26).  The rounding of
// Q moves a token's score by at most sum_j |c_j| 2^(e-27) scale, i.e. by at
// most 2^-22 of the token's own magnitude sum_j |qt_j c_j| scale when the
// codes are saturated at +-7.  Lane l then takes kv-head l % 8 of a group of kSalsHeads and
// token slot l / 8; a wave scores its two blocks together: per 64-token pass it
// reads the page-table entries of its 16 tokens, then their code words and
// scales (the 8 lanes of a slot read one token's 64 contiguous bytes), and
// folds each block's 8 scores per lane into a base-2 (max, sum).  The 8 token
// slots of a kv-head are merged by three lane exchanges (xor 8, 16, 32).
// (sixteen query rows of fp32 need more registers: three waves per SIMD)
template <int QT, int G>
__global__ __launch_bounds__(256, G >= 16 ? 3 : 4) void sals_score_kernel(
    const void* __restrict__ q, int hq, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const float* __restrict__ proj, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    int unit_tokens, float tau_log2e, float* __restrict__ scores, int max_units) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ float sals_smem[];   // sized by sals_smem_bytes(hkv)
  float* proj_s = sals_smem;                      // [d][rank]
  float* qbar = proj_s + kHeadDim * kRank;        // [hkv][kQbarStride] group-mean query
  // [hkv][kQDigits][2] digit words of the projected index query (columns 0-7,
  // 8-15), then [hkv] scales 2^(e-26)
  uint32_t* qd_s = reinterpret_cast<uint32_t*>(qbar + hkv * kQbarStride);
  float* qf_s = reinterpret_cast<float*>(qd_s + hkv * 2 * kQDigits);
  const int b = blockIdx.y;
  const int L = clamp_len(lens[b], max_pages);
  const int nu = (L + unit_tokens - 1) / unit_tokens;
  const int u0 = blockIdx.x * kSalsUnitsPerWG;
  if (u0 >= nu) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = lane & (kSalsHeads - 1), ts = lane / kSalsHeads;
  const int32_t* pt_b = pt + (size_t)b * max_pages;
  const uint2* cw_base = reinterpret_cast<const uint2*>(codes);
  const int u_end = min(u0 + kSalsUnitsPerWG, nu);
  const int ua = u0 + wave;  // the wave's two blocks: ua and ua + 4

  // one pass = 64 tokens of both blocks for one group of kSalsHeads kv-heads
  int pp[16], tok[16];
  bool in[16], ok[16];
  uint2 cw[16];
  uint16_t sw[16];
  auto issue_pt = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = ua + 4 * (i / 8);
      const int to = t0 + ts + 8 * (i % 8);
      tok[i] = u * unit_tokens + to;
      in[i] = u < u_end && to < unit_tokens && tok[i] < L;
      pp[i] = pt_b[in[i] ? tok[i] >> 4 : 0];
    }
  };
  auto issue_codes = [&](int hh) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ok[i] = in[i] && pp[i] >= 0 && pp[i] < num_pages;
      const size_t row = ((size_t)(ok[i] ? pp[i] : 0) * kPage + (tok[i] & 15)) * hkv + hh;
      cw[i] = cw_base[row];
      sw[i] = scales[row];
    }
  };
  // the first pass's page-table entries, then (below) its codes, are in flight
  // while the index query is formed
  issue_pt(0);

  // P and the group means of q into LDS: four dimensions of one kv-head per
  // thread and item, its G query rows loaded at once, in the same round trip
  // as the page-table entries.  The codes of the first pass are issued next,
  // so they are in flight while qt is formed.
  {
    constexpr int kP4 = kHeadDim * kRank / 4 / 256;
    constexpr int kItemsPerHead = kHeadDim / 4;
    const int n_items = hkv * kItemsPerHead;
    const float inv_g = 1.0f / (float)G;
    auto load_item = [&](int pi, float4 (&qv)[G]) {
      const int hh = pi / kItemsPerHead, d0 = 4 * (pi % kItemsPerHead);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const size_t qi = ((size_t)b * hq + (size_t)hh * G + g) * kHeadDim + d0;
        if constexpr (QT == SA_F32) {
          qv[g] = *reinterpret_cast<const float4*>(static_cast<const float*>(q) + qi);
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + qi);
          qv[g] = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
        }
      }
    };
    auto store_item = [&](int pi, const float4 (&qv)[G]) {
      float4 sum = qv[0];
#pragma unroll
      for (int g = 1; g < G; ++g) {
        sum.x += qv[g].x;
        sum.y += qv[g].y;
        sum.z += qv[g].z;
        sum.w += qv[g].w;
      }
      float* dst = qbar + (pi / kItemsPerHead) * kQbarStride + 4 * (pi % kItemsPerHead);
      dst[0] = sum.x * inv_g;
      dst[1] = sum.y * inv_g;
      dst[2] = sum.z * inv_g;
      dst[3] = sum.w * inv_g;
    };
    float4 pv[kP4];
#pragma unroll
    for (int r = 0; r < kP4; ++r) pv[r] = reinterpret_cast<const float4*>(proj)[tid + 256 * r];
    float4 qv[G];
    if (tid < n_items) load_item(tid, qv);
#pragma unroll
    for (int r = 0; r < kP4; ++r) reinterpret_cast<float4*>(proj_s)[tid + 256 * r] = pv[r];
    if (tid < n_items) store_item(tid, qv);
    for (int pi = tid + 256; pi < n_items; pi += 256) {
      load_item(pi, qv);
      store_item(pi, qv);
    }
  }
  // nothing above may sink below the code loads: a load issued after them
  // would wait for them (memory counters retire in order)
  __builtin_amdgcn_sched_barrier(0);
  issue_codes(x < hkv ? x : 0);
  __syncthreads();
  for (int t = wave; t * 16 < hkv; t += 4) {  // qt rows 16 t .. 16 t + 15
    // rows past hkv repeat the last kv-head; their results are not used
    const int m = min(16 * t + (lane & 15), hkv - 1);
    f32x4 c2[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll 8
    for (int kk = 0; kk < kHeadDim / 4; ++kk) {
      const int kx = 4 * kk + (lane >> 4);
      c2[kk & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(qbar[m * kQbarStride + kx],
                                                        proj_s[kx * kRank + (lane & 15)], c2[kk & 1], 0, 0, 0);
    }
    const f32x4 c = c2[0] + c2[1];
    // row 16 t + 4 (lane / 16) + i, column j = lane % 16: the scale exponent
    // from the row max, then each digit's nibble, OR-combined over the eight
    // columns of a word
    const int j = lane & 15;
    int ex[4];
    uint32_t w[4][kQDigits];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      (void)frexpf(max16(fabsf(c[i])), &ex[i]);
      const uint32_t u = (uint32_t)((int)rintf(ldexpf(c[i], kQFracBits - ex[i])) + 0x8888888);
#pragma unroll
      for (int k = 0; k < kQDigits; ++k) w[i][k] = (((u >> (4 * k)) & 15u) ^ 8u) << (4 * (j & 7));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < kQDigits; ++k) w[i][k] |= dpp_u32<kDppXor1>(w[i][k]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < kQDigits; ++k) w[i][k] |= dpp_u32<kDppXor2>(w[i][k]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < kQDigits; ++k) w[i][k] |= dpp_u32<kDppHalfMirror>(w[i][k]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * t + 4 * (lane >> 4) + i;
      if (row < hkv && (j & 7) == 0) {
#pragma unroll
        for (int k = 0; k < kQDigits; ++k) qd_s[(row * kQDigits + k) * 2 + (j >> 3)] = w[i][k];
      }
      if (row < hkv && j == 0) qf_s[row] = ldexpf(1.0f, ex[i] - kQFracBits);
    }
  }
  __syncthreads();

  for (int h0 = 0; h0 < hkv; h0 += kSalsHeads) {
    const bool hv = h0 + x < hkv;
    const int hh = hv ? h0 + x : h0;
    uint2 qd[kQDigits];
#pragma unroll
    for (int k = 0; k < kQDigits; ++k) qd[k] = reinterpret_cast<const uint2*>(qd_s)[hh * kQDigits + k];
    const float fz = tau_log2e * qf_s[hh];
    float m[2] = {-INFINITY, -INFINITY}, s[2] = {0.0f, 0.0f};
    for (int t0 = 0; t0 < unit_tokens; t0 += 64) {
      if (h0 > 0 || t0 > 0) {  // the first pass was fetched ahead
        issue_pt(t0);
        issue_codes(hh);
      }
      // sum_j c_j Q_j per token: Horner over the high digits (|.| < 7 * 16 *
      // 0x888) and over the low digits (|.| < 7 * 16 * 0x8888), each exact in
      // int32 and in fp32, then hi * 16^4 + lo with one rounding; the 16
      // tokens interleaved
      int dot[16];
      float dotf[16];
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) dot[ii] = 0;
#pragma unroll
      for (int k = kQDigits - 1; k >= kQLoDigits; --k) {
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          dot[ii] = __builtin_amdgcn_sdot8((int)cw[ii].x, (int)qd[k].x, dot[ii], false);
          dot[ii] = __builtin_amdgcn_sdot8((int)cw[ii].y, (int)qd[k].y, dot[ii], false);
          if (k > kQLoDigits) dot[ii] = (int)((uint32_t)dot[ii] << 4);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        dotf[ii] = (float)dot[ii];
        dot[ii] = 0;
      }
#pragma unroll
      for (int k = kQLoDigits - 1; k >= 0; --k) {
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          dot[ii] = __builtin_amdgcn_sdot8((int)cw[ii].x, (int)qd[k].x, dot[ii], false);
          dot[ii] = __builtin_amdgcn_sdot8((int)cw[ii].y, (int)qd[k].y, dot[ii], false);
          if (k > 0) dot[ii] = (int)((uint32_t)dot[ii] << 4);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) dotf[ii] = fmaf(dotf[ii], 65536.0f, (float)dot[ii]);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float z[8], zmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int ii = 8 * blk + i;
          const float zv = fz * (f16_to_f32(sw[ii]) * dotf[ii]);
          z[i] = (ok[ii] && hv) ? zv : -INFINITY;
          zmax = fmaxf(zmax, z[i]);
        }
        if (zmax != -INFINITY) {
          float sc = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) sc += z[i] == -INFINITY ? 0.0f : exp2f(z[i] - zmax);
          lse_merge(m[blk], s[blk], zmax, sc);
        }
      }
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // the 8 token slots of kv-head x: lanes x + 8 k
      float mb = m[blk], sb = s[blk];
      auto ror8 = [](float v) {  // DPP row_ror:8
        return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x128, 0xF, 0xF,
                                                                     false));
      };
      lse_merge(mb, sb, ror8(mb), ror8(sb));
      {
        const auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
        const auto rs = __builtin_amdgcn_permlane16_swap(__float_as_uint(sb), __float_as_uint(sb), false, false);
        mb = __uint_as_float(rm[0]);
        sb = __uint_as_float(rs[0]);
        lse_merge(mb, sb, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
      }
      {
        const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(mb), __float_as_uint(mb), false, false);
        const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(sb), __float_as_uint(sb), false, false);
        mb = __uint_as_float(rm[0]);
        sb = __uint_as_float(rs[0]);
        lse_merge(mb, sb, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
      }
      const int u = ua + 4 * blk;
      if (ts == 0 && hv && u < u_end)
        scores[((size_t)b * hkv + h0 + x) * max_units + u] = mb == -INFINITY ? -INFINITY : (mb + __log2f(sb)) * kLn2;
    }
  }
}

constexpr int kProbeUnitsPerWave = 4;
constexpr int kProbeUnitsPerWG = 4 * kProbeUnitsPerWave;

// Probe sampling [RK, the probe signal of the block selector]: the score of
// block u is the largest q_g . k_t over its probed positions t (step =
// max(1, len / n_probe) from the block start) and the group's query heads g.
// grid (ceil(max_units / 16), Hkv, B), block 256: the group's query rows are
// staged in LDS as fp32; wave w takes the four consecutive blocks from
// (blockIdx.x * 4 + w) * 4, with the page-table entries and then the key rows
// of all four in flight together (one block per wave left each wave a chain of
// dependent round trips for 2 KB of keys).  Lanes are (probe slot of 8,
// dimension group of 8 x 16): each round reads up to eight probed key rows per
// block (16 dimensions per lane), sums each slot's partial dots over its eight
// lanes by DPP, and keeps the maximum; the eight slots are merged by a row
// maximum and two lane swaps.  int8 keys: the dot of the codes times the
// token's scale.
template <int KT, int QT, int G>
__global__ __launch_bounds__(256) void probe_score_kernel(
    const void* __restrict__ q, int hq, const void* __restrict__ k,
    const uint16_t* __restrict__ k_scale, int num_pages, int hkv, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ lens, int max_pages, int unit_tokens, int n_probe,
    float* __restrict__ scores, int max_units) {
  constexpr int UPW = kProbeUnitsPerWave;
  __shared__ float qs[G][kHeadDim];
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const size_t qi = ((size_t)b * hq + (size_t)h * G + i / kHeadDim) * kHeadDim + i % kHeadDim;
    qs[i / kHeadDim][i % kHeadDim] = QT == SA_F32 ? static_cast<const float*>(q)[qi]
                                                  : bf16_to_f32(static_cast<const uint16_t*>(q)[qi]);
  }
  __syncthreads();
  const int L = clamp_len(lens[b], max_pages);
  const int nu = (L + unit_tokens - 1) / unit_tokens;
  const int ub = (blockIdx.x * 4 + wave) * UPW;
  if (ub >= nu) return;  // wave-uniform, and no barrier follows
  int t0[UPW], stp[UPW], ns[UPW];
  int ns_max = 0;
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = ub + j;
    t0[j] = 0;
    stp[j] = 1;
    ns[j] = 0;  // blocks past the sequence probe nothing
    if (u < nu) {
      t0[j] = u * unit_tokens;
      const int t1 = min(t0[j] + unit_tokens, L);
      stp[j] = max(1, (t1 - t0[j]) / n_probe);
      ns[j] = (t1 - t0[j] + stp[j] - 1) / stp[j];
    }
    ns_max = max(ns_max, ns[j]);
  }
  const int slot = lane >> 3, dg = lane & 7;
  const int32_t* pt_row = pt + (size_t)b * max_pages;
  float best[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) best[j] = -INFINITY;
  for (int i0 = 0; i0 < ns_max; i0 += 8) {
    const int i = i0 + slot;
    int pp[UPW], t[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      t[j] = t0[j] + (i < ns[j] ? i : 0) * stp[j];
      pp[j] = pt_row[t[j] >> 4];
    }
    bool ok[UPW];
    float x[UPW][16], sc[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      ok[j] = i < ns[j] && pp[j] >= 0 && pp[j] < num_pages;
      const size_t row = ((size_t)(ok[j] ? pp[j] : 0) * kPage + (t[j] & 15)) * hkv + h;
      float a[8], c[8];
      load8<KT>(k, row * kHeadDim + 16 * dg, a);
      load8<KT>(k, row * kHeadDim + 16 * dg + 8, c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[j][e] = a[e];
        x[j][8 + e] = c[e];
      }
      sc[j] = KT == SA_I8 ? f16_to_f32(k_scale[row]) : 1.0f;
    }
    constexpr int GU = G > 4 ? 2 : G;  // larger groups: query rows re-read from LDS, not held
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
#pragma unroll GU
      for (int g = 0; g < G; ++g) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) dot = fmaf(qs[g][16 * dg + e], x[j][e], dot);
        dot += dpp_f32<kDppXor1>(dot);
        dot += dpp_f32<kDppXor2>(dot);
        dot += dpp_f32<kDppHalfMirror>(dot);
        if (ok[j]) best[j] = fmaxf(best[j], dot * sc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const float bj = pair32_max(pair16_max(max16(best[j])));
    if (lane == 0 && ub + j < nu) scores[((size_t)b * hkv + h) * max_units + ub + j] = bj;
  }
}

template <int KT, int QT, bool PH>
hipError_t quest_dispatch_g(int G, dim3 grid, hipStream_t st, const void* q, const void* meta,
                            const Shapes& s, const int32_t* pt, const int32_t* lens,
                            float* scores) {
#define SA_QS(GG)                                                                              \
  hipLaunchKernelGGL((quest_score_kernel<KT, QT, GG, PH>), grid, dim3(256), 0, st, q, meta,    \
                     s.num_pages, s.Hkv, pt, lens, s.max_pages, scores)
  switch (G) {
    case 1: SA_QS(1); break;
    case 2: SA_QS(2); break;
    case 4: SA_QS(4); break;
    case 8: SA_QS(8); break;
    default: SA_QS(16); break;
  }
#undef SA_QS
  return hipGetLastError();
}

template <int KT, int QT>
hipError_t quest_dispatch(bool per_head, int G, dim3 grid, hipStream_t st, const void* q,
                          const void* meta, const Shapes& s, const int32_t* pt,
                          const int32_t* lens, float* scores) {
  return per_head ? quest_dispatch_g<KT, QT, true>(G, grid, st, q, meta, s, pt, lens, scores)
                  : quest_dispatch_g<KT, QT, false>(G, grid, st, q, meta, s, pt, lens, scores);
}

}  // namespace

hipError_t launch_quest_score(int kv_dtype, int q_dtype, const void* q, const void* meta,
                              const Shapes& s, const int32_t* pt, const int32_t* lens,
                              float* scores, hipStream_t st, bool per_head) {
  const int G = s.Hq / s.Hkv;
  dim3 grid((s.max_pages + kScorePagesPerWG - 1) / kScorePagesPerWG, s.Hkv, s.B);
  if (kv_dtype == SA_F32)
    return q_dtype == SA_F32 ? quest_dispatch<SA_F32, SA_F32>(per_head, G, grid, st, q, meta, s, pt, lens, scores)
                             : quest_dispatch<SA_F32, SA_BF16>(per_head, G, grid, st, q, meta, s, pt, lens, scores);
  if (q_dtype == SA_BF16 && G >= 4) {  // bf16 query groups of four or more: matrix cores
    const dim3 gm((s.max_pages + kMfmaPagesPerWG - 1) / kMfmaPagesPerWG, s.Hkv, s.B);
    const uint16_t* qh = static_cast<const uint16_t*>(q);
    const uint16_t* mh = static_cast<const uint16_t*>(meta);
#define SA_QM(GG, PH)                                                                               \
  hipLaunchKernelGGL((quest_score_mfma_kernel<GG, PH>), gm, dim3(256), 0, st, qh, mh, s.num_pages, \
                     s.Hkv, pt, lens, s.max_pages, scores)
#define SA_QMG(PH)                  \
  switch (G) {                      \
    case 4: SA_QM(4, PH); break;    \
    case 8: SA_QM(8, PH); break;    \
    default: SA_QM(16, PH); break;  \
  }
    if (per_head) {
      SA_QMG(true)
    } else {
      SA_QMG(false)
    }
#undef SA_QMG
#undef SA_QM
    return hipGetLastError();
  }
  return q_dtype == SA_F32 ? quest_dispatch<SA_BF16, SA_F32>(per_head, G, grid, st, q, meta, s, pt, lens, scores)
                           : quest_dispatch<SA_BF16, SA_BF16>(per_head, G, grid, st, q, meta, s, pt, lens, scores);
}

hipError_t launch_sals_score(int q_dtype, const void* q, const uint8_t* codes,
                             const uint16_t* scales, const float* proj, const Shapes& s,
                             const int32_t* pt, const int32_t* lens, int unit_tokens, float tau,
                             float* scores, int max_units, hipStream_t st) {
  dim3 grid((max_units + kSalsUnitsPerWG - 1) / kSalsUnitsPerWG, s.B);
  const float tl2 = tau * kLog2e;
  const size_t smem = sals_smem_bytes(s.Hkv);
#define SA_SS(QQ, GG)                                                                            \
  hipLaunchKernelGGL((sals_score_kernel<QQ, GG>), grid, dim3(256), smem, st, q, s.Hq, codes,     \
                     scales, proj, s.num_pages, s.Hkv, pt, lens, s.max_pages, unit_tokens, tl2,  \
                     scores, max_units)
#define SA_SG(QQ)                     \
  switch (s.Hq / s.Hkv) {             \
    case 1: SA_SS(QQ, 1); break;      \
    case 2: SA_SS(QQ, 2); break;      \
    case 4: SA_SS(QQ, 4); break;      \
    case 8: SA_SS(QQ, 8); break;      \
    default: SA_SS(QQ, 16); break;    \
  }
  if (q_dtype == SA_F32) {
    SA_SG(SA_F32)
  } else {
    SA_SG(SA_BF16)
  }
#undef SA_SG
#undef SA_SS
  return hipGetLastError();
}

hipError_t launch_probe_score(int kv_dtype, int q_dtype, const void* q, const void* k,
                              const uint16_t* k_scale, const Shapes& s, const int32_t* pt,
                              const int32_t* lens, int unit_tokens, int n_probe, float* scores,
                              int max_units, hipStream_t st) {
  const dim3 grid((max_units + kProbeUnitsPerWG - 1) / kProbeUnitsPerWG, s.Hkv, s.B);
#define SA_PR(KT, QT, GG)                                                                       \
  hipLaunchKernelGGL((probe_score_kernel<KT, QT, GG>), grid, dim3(256), 0, st, q, s.Hq, k,      \
                     k_scale, s.num_pages, s.Hkv, pt, lens, s.max_pages, unit_tokens, n_probe,  \
                     scores, max_units)
#define SA_PR_G(KT, QT)                 \
  switch (s.Hq / s.Hkv) {               \
    case 1: SA_PR(KT, QT, 1); break;    \
    case 2: SA_PR(KT, QT, 2); break;    \
    case 4: SA_PR(KT, QT, 4); break;    \
    case 8: SA_PR(KT, QT, 8); break;    \
    default: SA_PR(KT, QT, 16); break;  \
  }
#define SA_PR_Q(KT)                          \
  if (q_dtype == SA_F32) {                   \
    SA_PR_G(KT, SA_F32)                      \
  } else {                                   \
    SA_PR_G(KT, SA_BF16)                     \
  }
  if (kv_dtype == SA_F32) {
    SA_PR_Q(SA_F32)
  } else if (kv_dtype == SA_BF16) {
    SA_PR_Q(SA_BF16)
  } else {
    SA_PR_Q(SA_I8)
  }
#undef SA_PR_Q
#undef SA_PR_G
#undef SA_PR
  return hipGetLastError();
}

}  // namespace sa
