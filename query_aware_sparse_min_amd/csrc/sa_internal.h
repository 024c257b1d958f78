// sa_internal.h - shared device helpers and launcher declarations of the
// gfx950 sparse decode-attention library.  Not a public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa.h"

namespace sa {

constexpr int kPage = 16;      // tokens per page
constexpr int kHeadDim = 128;  // head dimension
constexpr int kRank = 16;      // SALS index-key width
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Eight consecutive elements of a K/V/metadata row as fp32 (exact widening).
// DT: SA_F32 | SA_BF16 | SA_I8 (int8 returns the integer codes as floats).
template <int DT>
__device__ __forceinline__ void load8(const void* base, size_t elem, float (&x)[8]) {
  if constexpr (DT == SA_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else if constexpr (DT == SA_BF16) {
    uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    uint2 w = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(base) + elem);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = (float)(int8_t)(w.x >> (8 * e));
      x[4 + e] = (float)(int8_t)(w.y >> (8 * e));
    }
  }
}

__device__ __forceinline__ int clamp_len(int L, int max_pages) {
  return L < 0 ? 0 : (L > max_pages * kPage ? max_pages * kPage : L);
}

// --------------------------------------------------------- wave reductions
// Cross-lane exchanges on the VALU (DPP row permutes and the gfx950
// permlane16/32 swaps) rather than LDS-crossbar permutes.  Every step pairs
// lanes symmetrically, so all lanes of a group end with bit-identical values.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each 16 lanes

// permlane16/32_swap exchange lane l's value with lane l ^ 16 / l ^ 32; of the
// two results one is the lane's own value and the other the partner's, so a
// commutative combine of both gives the pair result.
__device__ __forceinline__ float sum16(float v) {  // all-reduce over each 16-lane row
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float pair16_sum(float v) {  // + lane l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {  // + lane l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max16(float v) {  // all-reduce max over each 16-lane row
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppXor1>(v));
  v = min(v, dpp_u32<kDppXor2>(v));
  v = min(v, dpp_u32<kDppHalfMirror>(v));
  v = min(v, dpp_u32<kDppMirror>(v));
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(b[0], b[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}
// Inclusive prefix sum over the 64 lanes (row shifts, then row broadcasts).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_shift_u32(uint32_t v) {  // invalid source lanes give 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_shift_u32<0x111, 0xF>(v);  // row_shr:1
  v += dpp_shift_u32<0x112, 0xF>(v);  // row_shr:2
  v += dpp_shift_u32<0x114, 0xF>(v);  // row_shr:4
  v += dpp_shift_u32<0x118, 0xF>(v);  // row_shr:8
  v += dpp_shift_u32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_shift_u32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// ------------------------------------------- cross-workgroup hand-off memory
// Data that one workgroup of a kernel writes and another reads in the same
// launch goes through device-coherent (sc1) stores and loads: the 8 XCD L2
// caches are not coherent with each other, and these accesses bypass stale
// copies without the whole-cache write-back / invalidate of an agent-scope
// fence.  COH = false gives plain accesses (hand-off across kernel launches).
template <bool COH, typename T>
__device__ __forceinline__ T ld_x(const T* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH, typename T>
__device__ __forceinline__ void st_x(T* p, T v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
// Order-preserving unsigned key of a score (-0.0 folded into +0.0).  Never 0
// for a non-NaN score, so 0 can mark a key that has not been written yet.
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0.0 -> +0.0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wait until this thread's stores have completed (s_waitcnt vmcnt(0)); the
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------------ launchers
// Every launcher enqueues on 'stream' and returns hipGetLastError() of the launch.
struct Shapes {
  int B, Hq, Hkv, max_pages, num_pages;
};

hipError_t launch_quest_meta(int dtype, const void* k, const Shapes& s, const int32_t* pt,
                             const int32_t* lens, void* meta, hipStream_t st);
hipError_t launch_sals_index(int dtype, const void* k, const uint16_t* k_scale, const Shapes& s,
                             const int32_t* pt, const int32_t* lens, const float* proj,
                             uint8_t* codes, uint16_t* scales, hipStream_t st);
hipError_t launch_append(int dtype, int mode, const void* k_new, const void* v_new,
                         const uint16_t* ks_new, const uint16_t* vs_new, void* k, void* v,
                         uint16_t* k_scale, uint16_t* v_scale, const Shapes& s, const int32_t* pt,
                         const int32_t* lens, const float* proj, void* meta, uint16_t* meta_scale,
                         hipStream_t st);
hipError_t launch_probe_score(int kv_dtype, int q_dtype, const void* q, const void* k,
                              const uint16_t* k_scale, const Shapes& s, const int32_t* pt,
                              const int32_t* lens, int unit_tokens, int n_probe, float* scores,
                              int max_units, hipStream_t st);
hipError_t launch_quest_score(int kv_dtype, int q_dtype, const void* q, const void* meta,
                              const Shapes& s, const int32_t* pt, const int32_t* lens,
                              float* scores, hipStream_t st, bool per_head = false);
hipError_t launch_sals_score(int q_dtype, const void* q, const uint8_t* codes,
                             const uint16_t* scales, const float* proj, const Shapes& s,
                             const int32_t* pt, const int32_t* lens, int unit_tokens, float tau,
                             float* scores, int max_units, hipStream_t st);
hipError_t launch_topk(const float* scores, int max_units, const Shapes& s, const int32_t* lens,
                       int unit_tokens, int k, int n_head, int n_tail, int32_t* sel,
                       int32_t* num_sel, int max_sel, hipStream_t st);

struct AttnPlan {
  int list_len;   // pages per (b, kv-head) list the kernel may visit
  int pps;        // pages per split
  int nsplit;     // splits per list
  int tasks;      // dense passes: workgroups of the device-planned launch (0: the host plan)
  size_t partial_floats;  // workspace floats
};
constexpr int kPlanMaxSeqs = 1024;  // sequences of a device-planned dense pass
// dense: a pass over every page of each sequence, split by the device plan
// from the actual lengths (B <= kPlanMaxSeqs)
AttnPlan plan_attention(int B, int Hq, int Hkv, int list_len, bool dense = false);

// Per-head selection: the union of a group's per-head page lists (ascending,
// (head mask << 16) | page entries, umax per list) for the masked attention.
constexpr int kUnionPages = 16384;  // largest max_pages the union supports
hipError_t launch_union(const int32_t* sel, const int32_t* num_sel, int max_sel, const Shapes& s,
                        const int32_t* lens, int32_t* ulist, int32_t* ucount, int umax,
                        hipStream_t st);

// Streaming read of bytes (a multiple of 16) at src by grid workgroups; sink
// holds grid words (written only in a case no realistic input reaches).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t st);

hipError_t launch_attention(int kv_dtype, int q_dtype, const void* q, const void* k,
                            const void* v, const uint16_t* k_scale, const uint16_t* v_scale,
                            const Shapes& s, const int32_t* pt, const int32_t* lens,
                            const int32_t* sel, const int32_t* num_sel, int max_sel,
                            const AttnPlan& plan, float softmax_scale, float* partials,
                            float* out, hipStream_t st, bool masked = false);

}  // namespace sa
