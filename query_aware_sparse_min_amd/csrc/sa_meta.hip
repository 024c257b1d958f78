// sa_meta.hip - selection metadata builders (amortised; run once per token
// insert or once per cache build, not inside the decode step).
//
//  * Quest min/max metadata ("Quest 完全拆解" explainer, page-level
//    management and the insert-time update M <- max(M, k), m <- min(m, k)):
//    one workgroup per referenced page; each thread owns 8 consecutive
//    (kv-head, dim) elements of the page's token rows and folds the page's
//    valid slots in order, so every load is a coalesced 16-byte row chunk and
//    the winner's bits are copied unchanged (exact, KV dtype).
//  * SALS int4 low-rank index key ("SALS长序列推理优化", low-rank preprocessing
//    and the int4 index key of QSI): one thread per (token, kv-head) runs the
//    16 fp32 fused-multiply-add chains k * P in dimension order, so its codes
//    are bit-identical to any other evaluation of the same definition.
//  * Decode-time append of one token per sequence: the token's K/V rows into
//    its page, then the same per-token metadata step (Quest: one more fold of
//    M <- max(M, k), m <- min(m, k); SALS: the token's index key), so the
//    metadata after any run of appends equals a full rebuild.
#pragma clang fp contract(off)

#include "sa_internal.h"

namespace sa {
namespace {

// An 8-element chunk of a row as raw 32-bit words: fp32 = 8 words, bf16 = 4.
template <int DT>
struct Chunk8 {
  static constexpr int W = DT == SA_F32 ? 8 : 4;
  uint32_t w[W];
  __device__ __forceinline__ void load(const void* p) {
    const uint4* q = static_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      uint4 t = q[i];
      w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
    }
  }
  __device__ __forceinline__ void store(void* p) const {
    uint4* q = static_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) q[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  }
  __device__ __forceinline__ uint32_t bits(int e) const {
    if constexpr (DT == SA_F32) return w[e];
    else return (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
  }
  __device__ __forceinline__ void set(int e, uint32_t b) {
    if constexpr (DT == SA_F32) w[e] = b;
    else w[e >> 1] = (w[e >> 1] & ~(0xffffu << (16 * (e & 1)))) | (b << (16 * (e & 1)));
  }
  __device__ __forceinline__ float val(int e) const {
    if constexpr (DT == SA_F32) return __uint_as_float(w[e]);
    else return __uint_as_float(bits(e) << 16);
  }
};

// grid (max_pages, B), block 256
template <int DT>
__global__ __launch_bounds__(256) void quest_meta_kernel(const void* __restrict__ k_,
                                                         int num_pages, int hkv,
                                                         const int32_t* __restrict__ pt,
                                                         const int32_t* __restrict__ lens,
                                                         int max_pages, void* __restrict__ meta_) {
  constexpr int ES = DT == SA_F32 ? 4 : 2;  // element bytes
  const int p = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(lens[b], max_pages);
  const int n = (L + kPage - 1) / kPage;
  if (p >= n) return;
  const int pp = pt[(size_t)b * max_pages + p];
  if (pp < 0 || pp >= num_pages) return;
  const int valid = min(kPage, L - p * kPage);
  const char* k = static_cast<const char*>(k_);
  char* meta = static_cast<char*>(meta_);
  const int row = hkv * kHeadDim;  // elements per token row
  const int chunks = row / 8;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const int h = c / (kHeadDim / 8);
    const int i0 = (c % (kHeadDim / 8)) * 8;
    const char* src = k + ((size_t)pp * kPage * row + (size_t)c * 8) * ES;
    Chunk8<DT> mx, mn;
    mx.load(src);
    mn = mx;
    float fmx[8], fmn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) fmx[e] = fmn[e] = mx.val(e);
    for (int s = 1; s < valid; ++s) {
      Chunk8<DT> v;
      v.load(src + (size_t)s * row * ES);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v.val(e);
        if (x > fmx[e]) { fmx[e] = x; mx.set(e, v.bits(e)); }
        if (x < fmn[e]) { fmn[e] = x; mn.set(e, v.bits(e)); }
      }
    }
    // head-major [Hkv][num_pages][2][d]: one list's records are contiguous
    mx.store(meta + ((((size_t)h * num_pages + pp) * 2 + 0) * kHeadDim + i0) * ES);
    mn.store(meta + ((((size_t)h * num_pages + pp) * 2 + 1) * kHeadDim + i0) * ES);
  }
}

// Index key of one (token, kv-head) row: key elements at k + e0 .. + d - 1
// (int8: codes times sc), P in LDS; writes the two code words and the scale.
template <int DT>
__device__ __forceinline__ void sals_key(const void* __restrict__ k, size_t e0, float sc,
                                         const float* P, uint2* crow, uint16_t* srow) {
  float acc[kRank];
#pragma unroll
  for (int j = 0; j < kRank; ++j) acc[j] = 0.0f;
  for (int i = 0; i < kHeadDim; i += 8) {
    float x[8];
    load8<DT>(k, e0 + i, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kh = (DT == SA_I8) ? x[e] * sc : x[e];  // int8: code * scale, exact in fp32
#pragma unroll
      for (int j = 0; j < kRank; ++j) acc[j] = __builtin_fmaf(kh, P[(i + e) * kRank + j], acc[j]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kRank; ++j) amax = fmaxf(amax, fabsf(acc[j]));
  const _Float16 sh = (_Float16)(amax / 7.0f);  // IEEE division, then RNE to fp16
  const float sf = (float)sh;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < kRank; ++j) {
    float c = 0.0f;
    if (sf != 0.0f) c = fminf(fmaxf(__builtin_rintf(acc[j] / sf), -7.0f), 7.0f);
    const uint32_t nib = (uint32_t)((int)c) & 0xFu;
    w[j / 8] |= nib << (4 * (j % 8));
  }
  *crow = make_uint2(w[0], w[1]);
  *srow = __builtin_bit_cast(uint16_t, sh);
}

// grid (max_pages, B), block 256; P staged in LDS (8 KiB)
template <int DT>
__global__ __launch_bounds__(256) void sals_index_kernel(
    const void* __restrict__ k, const uint16_t* __restrict__ k_scale, int num_pages, int hkv,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens, int max_pages,
    const float* __restrict__ proj, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  __shared__ float P[kHeadDim * kRank];
  const int p = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(lens[b], max_pages);
  const int n = (L + kPage - 1) / kPage;
  if (p >= n) return;
  const int pp = pt[(size_t)b * max_pages + p];
  if (pp < 0 || pp >= num_pages) return;
  for (int i = threadIdx.x; i < kHeadDim * kRank; i += blockDim.x) P[i] = proj[i];
  __syncthreads();
  for (int r = threadIdx.x; r < kPage * hkv; r += blockDim.x) {
    const int slot = r / hkv, h = r % hkv;
    const size_t row = ((size_t)pp * kPage + slot) * hkv + h;
    uint2* crow = reinterpret_cast<uint2*>(codes + row * (kRank / 2));
    if (p * kPage + slot >= L) {
      *crow = make_uint2(0u, 0u);
      scales[row] = 0;
      continue;
    }
    float sc = 1.0f;
    if constexpr (DT == SA_I8) sc = f16_to_f32(k_scale[row]);
    sals_key<DT>(k, row * kHeadDim, sc, P, crow, scales + row);
  }
}

// grid (B), block 256: one new token per sequence, at t = lens[b] - 1.  Its
// K/V rows (and int8 scales) are copied into slot t % 16 of its page, then
// the page's metadata takes the token: QUEST folds it into (M, m) with the
// comparisons quest_meta_kernel folds with (slot 0 starts the page); SALS
// writes the token's index key, computed as sals_key does.  META: 0 = no
// metadata (probe sampling reads K itself), 1 = QUEST, 2 = SALS.
template <int DT, int META>
__global__ __launch_bounds__(256) void append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const uint16_t* __restrict__ ks_new, const uint16_t* __restrict__ vs_new, void* k_, void* v_,
    uint16_t* k_scale, uint16_t* v_scale, int num_pages, int hkv, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ lens, int max_pages, const float* __restrict__ proj, void* meta_,
    uint16_t* meta_scale) {
  constexpr int ES = DT == SA_F32 ? 4 : DT == SA_BF16 ? 2 : 1;  // element bytes
  constexpr bool SALS = META == 2;
  __shared__ float P[SALS ? kHeadDim * kRank : 1];
  const int b = blockIdx.x;
  const int L = lens[b];
  if (L < 1 || L > max_pages * kPage) return;
  const int t = L - 1, slot = t % kPage;
  const int pp = pt[(size_t)b * max_pages + t / kPage];
  if (pp < 0 || pp >= num_pages) return;
  const int row = hkv * kHeadDim;  // elements per token row
  const size_t src = (size_t)b * row, dst = ((size_t)pp * kPage + slot) * row;
  // K / V rows, 16 bytes per thread and step
  const int row16 = row * ES / 16;
  for (int c = threadIdx.x; c < row16; c += blockDim.x) {
    reinterpret_cast<uint4*>(static_cast<char*>(k_) + dst * ES)[c] =
        reinterpret_cast<const uint4*>(static_cast<const char*>(k_new) + src * ES)[c];
    reinterpret_cast<uint4*>(static_cast<char*>(v_) + dst * ES)[c] =
        reinterpret_cast<const uint4*>(static_cast<const char*>(v_new) + src * ES)[c];
  }
  if constexpr (DT == SA_I8) {
    for (int h = threadIdx.x; h < hkv; h += blockDim.x) {
      k_scale[((size_t)pp * kPage + slot) * hkv + h] = ks_new[(size_t)b * hkv + h];
      v_scale[((size_t)pp * kPage + slot) * hkv + h] = vs_new[(size_t)b * hkv + h];
    }
  }
  if constexpr (SALS) {
    for (int i = threadIdx.x; i < kHeadDim * kRank; i += blockDim.x) P[i] = proj[i];
    __syncthreads();
    // one 16-lane row per kv-head, lane j running output j's chain: the same
    // fmaf order, maximum, scale and codes as sals_key, sixteen chains wide
    const int j = threadIdx.x & 15;
    for (int h = threadIdx.x >> 4; h < hkv; h += blockDim.x >> 4) {
      const float sc = DT == SA_I8 ? f16_to_f32(ks_new[(size_t)b * hkv + h]) : 1.0f;
      float acc = 0.0f;
      for (int i = 0; i < kHeadDim; i += 8) {
        float x[8];
        load8<DT>(k_new, src + (size_t)h * kHeadDim + i, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kh = (DT == SA_I8) ? x[e] * sc : x[e];
          acc = __builtin_fmaf(kh, P[(i + e) * kRank + j], acc);
        }
      }
      const float amax = max16(fabsf(acc));
      const _Float16 sh = (_Float16)(amax / 7.0f);  // IEEE division, then RNE to fp16
      const float sf = (float)sh;
      const float c = sf != 0.0f ? fminf(fmaxf(__builtin_rintf(acc / sf), -7.0f), 7.0f) : 0.0f;
      uint32_t w = ((uint32_t)((int)c) & 0xFu) << (4 * (j & 7));
      w |= dpp_u32<kDppXor1>(w);
      w |= dpp_u32<kDppXor2>(w);
      w |= dpp_u32<kDppHalfMirror>(w);
      const size_t r = ((size_t)pp * kPage + slot) * hkv + h;
      if ((j & 7) == 0) reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(meta_) + r * (kRank / 2))[j >> 3] = w;
      if (j == 0) meta_scale[r] = __builtin_bit_cast(uint16_t, sh);
    }
  } else if constexpr (META == 1 && DT != SA_I8) {
    char* meta = static_cast<char*>(meta_);
    for (int c = threadIdx.x; c < row / 8; c += blockDim.x) {
      const int h = c / (kHeadDim / 8), i0 = (c % (kHeadDim / 8)) * 8;
      Chunk8<DT> x;
      x.load(static_cast<const char*>(k_new) + (src + (size_t)c * 8) * ES);
      char* mxp = meta + ((((size_t)h * num_pages + pp) * 2 + 0) * kHeadDim + i0) * ES;
      char* mnp = meta + ((((size_t)h * num_pages + pp) * 2 + 1) * kHeadDim + i0) * ES;
      Chunk8<DT> mx = x, mn = x;
      if (slot > 0) {
        mx.load(mxp);
        mn.load(mnp);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = x.val(e);
          if (xv > mx.val(e)) mx.set(e, x.bits(e));
          if (xv < mn.val(e)) mn.set(e, x.bits(e));
        }
      }
      mx.store(mxp);
      mn.store(mnp);
    }
  }
}

}  // namespace

hipError_t launch_quest_meta(int dtype, const void* k, const Shapes& s, const int32_t* pt,
                             const int32_t* lens, void* meta, hipStream_t st) {
  dim3 grid(s.max_pages, s.B);
  if (dtype == SA_F32)
    hipLaunchKernelGGL(quest_meta_kernel<SA_F32>, grid, dim3(256), 0, st, k, s.num_pages, s.Hkv,
                       pt, lens, s.max_pages, meta);
  else
    hipLaunchKernelGGL(quest_meta_kernel<SA_BF16>, grid, dim3(256), 0, st, k, s.num_pages, s.Hkv,
                       pt, lens, s.max_pages, meta);
  return hipGetLastError();
}

hipError_t launch_sals_index(int dtype, const void* k, const uint16_t* k_scale, const Shapes& s,
                             const int32_t* pt, const int32_t* lens, const float* proj,
                             uint8_t* codes, uint16_t* scales, hipStream_t st) {
  dim3 grid(s.max_pages, s.B);
  switch (dtype) {
    case SA_F32:
      hipLaunchKernelGGL(sals_index_kernel<SA_F32>, grid, dim3(256), 0, st, k, k_scale,
                         s.num_pages, s.Hkv, pt, lens, s.max_pages, proj, codes, scales);
      break;
    case SA_BF16:
      hipLaunchKernelGGL(sals_index_kernel<SA_BF16>, grid, dim3(256), 0, st, k, k_scale,
                         s.num_pages, s.Hkv, pt, lens, s.max_pages, proj, codes, scales);
      break;
    default:
      hipLaunchKernelGGL(sals_index_kernel<SA_I8>, grid, dim3(256), 0, st, k, k_scale,
                         s.num_pages, s.Hkv, pt, lens, s.max_pages, proj, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_append(int dtype, int mode, const void* k_new, const void* v_new,
                         const uint16_t* ks_new, const uint16_t* vs_new, void* k, void* v,
                         uint16_t* k_scale, uint16_t* v_scale, const Shapes& s, const int32_t* pt,
                         const int32_t* lens, const float* proj, void* meta, uint16_t* meta_scale,
                         hipStream_t st) {
#define SA_AP(DT, META)                                                                          \
  hipLaunchKernelGGL((append_kernel<DT, META>), dim3(s.B), dim3(256), 0, st, k_new, v_new, ks_new, \
                     vs_new, k, v, k_scale, v_scale, s.num_pages, s.Hkv, pt, lens, s.max_pages,   \
                     proj, meta, meta_scale)
#define SA_AP_M(DT)                                     \
  switch (mode) {                                       \
    case SA_MODE_QUEST: SA_AP(DT, 1); break;            \
    case SA_MODE_SALS: SA_AP(DT, 2); break;             \
    default: SA_AP(DT, 0);                              \
  }
  switch (dtype) {
    case SA_F32: SA_AP_M(SA_F32) break;
    case SA_BF16: SA_AP_M(SA_BF16) break;
    default:  // QUEST metadata is not kept for int8 caches
      if (mode == SA_MODE_SALS) SA_AP(SA_I8, 2); else SA_AP(SA_I8, 0);
  }
#undef SA_AP_M
#undef SA_AP
  return hipGetLastError();
}

}  // namespace sa
