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
    float acc[kRank];
#pragma unroll
    for (int j = 0; j < kRank; ++j) acc[j] = 0.0f;
    for (int i = 0; i < kHeadDim; i += 8) {
      float x[8];
      load8<DT>(k, row * kHeadDim + i, x);
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
    scales[row] = __builtin_bit_cast(uint16_t, sh);
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

}  // namespace sa
