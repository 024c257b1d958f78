// sa_api.hip - the extern "C" boundary: argument validation, buffer sizing and
// launch planning, then the kernels of sa_meta / sa_score / sa_topk / sa_attn.
// Every check runs on the host before anything is enqueued, and no function
// allocates, frees or synchronises.
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "sa_internal.h"
#include "sa_post.h"
#include "sa_step.h"

using namespace sa;

// Scratch of sa_sparse_decode_attn_noalloc: the split-K partial records of one
// call, in device memory the library holds itself (each GPU the library runs
// on keeps its own copy until the process ends).  Every record is written by
// the attention kernel before the merge kernel reads it, so nothing in it has
// to start at zero.  In host code `scratch` is only a stand-in for the device
// symbol: the per-device address comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

// This device's copy of scratch, looked up once per device (with it current).
float* scratch_of_device() {
  static std::atomic<float*> cache[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  float* p = cache[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
  p = static_cast<float*>(addr);
  cache[dev].store(p, std::memory_order_release);
  return p;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_kv(const sa_kv_cache* kv) {
  if (!kv || !kv->k || !kv->v) return SA_ERR_INVALID_ARG;
  if (kv->dtype != SA_F32 && kv->dtype != SA_BF16 && kv->dtype != SA_I8) return SA_ERR_INVALID_ARG;
  if (kv->dtype == SA_I8 && (!kv->k_scale || !kv->v_scale)) return SA_ERR_INVALID_ARG;
  if (kv->num_pages < 1 || kv->num_kv_heads < 1 || kv->num_kv_heads > 65535) return SA_ERR_INVALID_ARG;
  if (kv->page_size != kPage || kv->head_dim != kHeadDim) return SA_ERR_UNSUPPORTED;
  if (!aligned16(kv->k) || !aligned16(kv->v)) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

int check_seqs(const sa_seqs* s) {
  if (!s || !s->page_table || !s->seq_lens) return SA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->batch > 65535 || s->max_pages < 1) return SA_ERR_INVALID_ARG;
  if ((long long)s->max_pages * kPage > 0x3FFFFFFFLL) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

// Fields that selection alone uses (sa_topk_pages, list sizes).
int check_select(const sa_select_cfg* c) {
  if (!c) return SA_ERR_INVALID_ARG;
  if (c->mode != SA_MODE_QUEST && c->mode != SA_MODE_SALS && c->mode != SA_MODE_PROBE)
    return SA_ERR_INVALID_ARG;
  if (c->k_compete < 0 || c->n_head_forced < 0 || c->n_tail_forced < 0) return SA_ERR_INVALID_ARG;
  if ((long long)c->k_compete + c->n_head_forced + c->n_tail_forced < 1) return SA_ERR_INVALID_ARG;
  if ((long long)c->k_compete + c->n_head_forced + c->n_tail_forced > 0x3FFFFFFLL) return SA_ERR_INVALID_ARG;
  if (c->unit_tokens < kPage || c->unit_tokens % kPage != 0) return SA_ERR_INVALID_ARG;
  if (c->mode == SA_MODE_QUEST && c->unit_tokens != kPage) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

// Everything scoring needs as well.
int check_cfg(const sa_select_cfg* c) {
  const int rc = check_select(c);
  if (rc != SA_OK) return rc;
  if (c->mode == SA_MODE_SALS) {
    if (!c->proj) return SA_ERR_INVALID_ARG;
    if (c->rank != kRank) return SA_ERR_UNSUPPORTED;
    if (!(c->lse_scale == c->lse_scale)) return SA_ERR_INVALID_ARG;  // NaN
  }
  if (c->mode == SA_MODE_PROBE && c->n_probe < 1) return SA_ERR_INVALID_ARG;
  if (c->per_head != 0 && c->per_head != 1) return SA_ERR_INVALID_ARG;
  if (c->per_head && c->mode != SA_MODE_QUEST) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

// query heads per kv-head supported by the kernels
bool group_ok(int hq, int hkv) {
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return false;
  const int G = hq / hkv;
  return G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
}

int check_q(const void* q, int q_dtype, int hq, int hkv) {
  if (!q || !aligned16(q)) return SA_ERR_INVALID_ARG;
  if (q_dtype != SA_F32 && q_dtype != SA_BF16) return SA_ERR_INVALID_ARG;
  if (hq < 1 || hq % hkv != 0) return SA_ERR_INVALID_ARG;
  if (!group_ok(hq, hkv)) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

int check_mode_kv(const sa_select_cfg* c, const sa_kv_cache* kv) {
  if (c->mode == SA_MODE_QUEST && kv->dtype == SA_I8) return SA_ERR_UNSUPPORTED;
  if (c->mode == SA_MODE_SALS && (64 % kv->num_kv_heads != 0)) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

int max_units_of(const sa_seqs* s, const sa_select_cfg* c) {
  return (int)(((long long)s->max_pages * kPage + c->unit_tokens - 1) / c->unit_tokens);
}

int max_sel_of(const sa_seqs* s, const sa_select_cfg* c) {
  const long long u = (long long)c->k_compete + c->n_head_forced + c->n_tail_forced;
  const long long pages = u * (c->unit_tokens / kPage);
  return (int)(pages < s->max_pages ? pages : s->max_pages);
}

int hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

Shapes shapes_of(int hq, const sa_kv_cache* kv, const sa_seqs* s) {
  return Shapes{s->batch, hq, kv->num_kv_heads, s->max_pages, kv->num_pages};
}

// Compute units of the current device (cached per device id).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Co-resident workgroups of the fused step kernel on the current device
// (0 when the kernel's build cannot show its residency: the separate kernels
// run instead), cached per (device, kv dtype, q dtype, keys per thread).
int resident_step_wgs(int kv_dtype, int q_dtype, int max_pages) {
  static std::atomic<int> cache[64][8];  // value + 1; 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int kpt = step_kpt(max_pages);
  const int slot = (kv_dtype == SA_F32 ? 0 : 2) + (q_dtype == SA_F32 ? 0 : 1) + (kpt > step_kpt(1) ? 4 : 0);
  if (dev < 64) {
    const int c = cache[dev][slot].load(std::memory_order_relaxed);
    if (c > 0) return c - 1;
  }
  const int n = step_resident_wgs(kv_dtype, q_dtype, kpt, device_cus());
  if (dev < 64) cache[dev][slot].store(n + 1, std::memory_order_relaxed);
  return n;
}

// Optional cap on the fused step kernel's workgroups: the environment variable
// SA_STEP_MAX_WORKGROUPS (a positive integer), read at every call; 0 = no cap.
int step_wg_cap() {
  const char* e = getenv("SA_STEP_MAX_WORKGROUPS");
  if (!e || !*e) return 0;
  const long v = strtol(e, nullptr, 10);
  return v > 0 && v < (1L << 20) ? (int)v : 0;
}

constexpr int kPlanCUs = 256;  // task decomposition is planned for a 256-CU MI355X

// Workspace of the per-head attention: the union lists and their lengths,
// then the split-K partial records over the union.
struct HeadsLayout {
  size_t ulist, ucount, partials, total;
  int umax;
  AttnPlan plan;
};

HeadsLayout heads_layout(int B, int hq, int hkv, int max_pages, int max_sel) {
  HeadsLayout H{};
  const long long u = (long long)(hq / hkv) * max_sel;
  H.umax = (int)(u < max_pages ? u : max_pages);
  if (H.umax < 1) H.umax = 1;
  H.plan = plan_attention(B, hq, hkv, H.umax);
  const size_t lists = (size_t)B * hkv;
  size_t off = 0;
  H.ulist = off;
  off = align_up(off + lists * H.umax * sizeof(int32_t));
  H.ucount = off;
  off = align_up(off + lists * sizeof(int32_t));
  H.partials = off;
  off = align_up(off + H.plan.partial_floats * sizeof(float));
  H.total = off;
  return H;
}

struct StepLayout {
  size_t arrive, scores, sel, num_sel, partials, heads, total;
  int max_units, max_sel;
  bool dense;  // every list keeps all of its units: no scoring needed
  bool fused;  // Quest: one persistent kernel for the whole step
  bool per_head;  // Quest: one selection per query head, attention over the group's union
  bool post;   // after the scorer: selection, attention and merge in one persistent kernel
  AttnPlan plan;
  StepPlan splan;
  PostPlan pplan;
  HeadsLayout hl;
};

StepLayout step_layout(int hq, const sa_kv_cache* kv, const sa_seqs* s, const sa_select_cfg* c,
                       int q_dtype) {
  StepLayout L{};
  L.max_units = max_units_of(s, c);
  L.max_sel = max_sel_of(s, c);
  L.dense = (long long)c->k_compete + c->n_head_forced + c->n_tail_forced >= L.max_units;
  L.per_head = c->per_head != 0 && !L.dense;
  L.fused = !L.dense && !L.per_head && c->mode == SA_MODE_QUEST &&
            hq / kv->num_kv_heads <= kStepMaxGroup && s->max_pages <= kStepMaxPages &&
            kv->num_pages <= kStepMaxPhysPages;
  // selection lists: one per kv-head, or one per query head with per_head
  const size_t lists = (size_t)s->batch * (L.per_head ? hq : kv->num_kv_heads);
  L.plan = plan_attention(s->batch, hq, kv->num_kv_heads, L.dense ? s->max_pages : L.max_sel,
                          L.dense);
  L.splan = plan_step(s->batch, hq, kv->num_kv_heads, s->max_pages, L.max_sel, kPlanCUs);
  const size_t fused_part = (size_t)L.splan.lists * L.splan.nc * (hq / kv->num_kv_heads) * (kHeadDim + 2);
  L.pplan = plan_post(L.splan.lists, hq / kv->num_kv_heads, L.max_sel, kPlanCUs);
  L.post = !L.dense && !L.per_head && !L.fused && L.pplan.ok &&
           post_supported(kv->dtype, q_dtype, hq / kv->num_kv_heads, L.max_units);
  const size_t post_part =
      L.post ? (size_t)L.pplan.lists * L.pplan.nc * (hq / kv->num_kv_heads) * (kHeadDim + 2) : 0;
  size_t off = 0;
  L.arrive = off;  // the fused kernel's per-list arrival counters
  off = align_up(off + (size_t)L.splan.lists * sizeof(uint32_t));
  L.scores = off;
  off = align_up(off + (L.dense ? 0 : lists * L.max_units * sizeof(float)));
  L.sel = off;
  off = align_up(off + lists * L.max_sel * sizeof(int32_t));
  L.num_sel = off;
  off = align_up(off + lists * sizeof(int32_t));
  L.partials = off;
  size_t pf = L.plan.partial_floats > fused_part ? L.plan.partial_floats : fused_part;
  if (post_part > pf) pf = post_part;
  off = align_up(off + pf * sizeof(float));
  L.heads = off;
  if (L.per_head) {
    L.hl = heads_layout(s->batch, hq, kv->num_kv_heads, s->max_pages, L.max_sel);
    off = align_up(off + L.hl.total);
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

int sa_version(void) { return 1; }

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t sa_meta_bytes(const sa_kv_cache* kv, const sa_select_cfg* cfg) {
  if (check_kv(kv) != SA_OK || check_cfg(cfg) != SA_OK) return 0;
  if (cfg->mode == SA_MODE_PROBE) return 0;
  if (cfg->mode == SA_MODE_QUEST) {
    if (kv->dtype == SA_I8) return 0;
    const size_t es = kv->dtype == SA_F32 ? 4 : 2;
    return (size_t)kv->num_pages * kv->num_kv_heads * 2 * kHeadDim * es;
  }
  return (size_t)kv->num_pages * kPage * kv->num_kv_heads * (kRank / 2);
}

size_t sa_meta_scale_bytes(const sa_kv_cache* kv, const sa_select_cfg* cfg) {
  if (check_kv(kv) != SA_OK || check_cfg(cfg) != SA_OK) return 0;
  if (cfg->mode != SA_MODE_SALS) return 0;
  return (size_t)kv->num_pages * kPage * kv->num_kv_heads * sizeof(uint16_t);
}

int32_t sa_max_units(const sa_seqs* seqs, const sa_select_cfg* cfg) {
  if (check_seqs(seqs) != SA_OK || check_select(cfg) != SA_OK) return 0;
  return max_units_of(seqs, cfg);
}

int32_t sa_max_selected(const sa_seqs* seqs, const sa_select_cfg* cfg) {
  if (check_seqs(seqs) != SA_OK || check_select(cfg) != SA_OK) return 0;
  return max_sel_of(seqs, cfg);
}

int sa_build_page_meta(const sa_kv_cache* kv, const sa_seqs* seqs, const sa_select_cfg* cfg,
                       void* meta, uint16_t* meta_scale, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs)) || (rc = check_cfg(cfg))) return rc;
  if ((rc = check_mode_kv(cfg, kv))) return rc;
  if (cfg->mode == SA_MODE_PROBE) return SA_OK;  // no metadata: the scores read K
  if (!meta || !aligned16(meta)) return SA_ERR_INVALID_ARG;
  const Shapes s = shapes_of(kv->num_kv_heads, kv, seqs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->mode == SA_MODE_QUEST)
    return hip_status(launch_quest_meta(kv->dtype, kv->k, s, seqs->page_table, seqs->seq_lens, meta, st));
  if (!meta_scale) return SA_ERR_INVALID_ARG;
  return hip_status(launch_sals_index(kv->dtype, kv->k, kv->k_scale, s, seqs->page_table,
                                      seqs->seq_lens, cfg->proj, static_cast<uint8_t*>(meta),
                                      meta_scale, st));
}

int sa_append_kv(const void* k_new, const void* v_new, const uint16_t* k_scale_new,
                 const uint16_t* v_scale_new, const sa_kv_cache* kv, const sa_seqs* seqs,
                 const sa_select_cfg* cfg, void* meta, uint16_t* meta_scale, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs)) || (rc = check_cfg(cfg))) return rc;
  if ((rc = check_mode_kv(cfg, kv))) return rc;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return SA_ERR_INVALID_ARG;
  if (kv->dtype == SA_I8 && (!k_scale_new || !v_scale_new)) return SA_ERR_INVALID_ARG;
  if (cfg->mode != SA_MODE_PROBE && (!meta || !aligned16(meta))) return SA_ERR_INVALID_ARG;
  if (cfg->mode == SA_MODE_SALS && !meta_scale) return SA_ERR_INVALID_ARG;
  const Shapes s = shapes_of(kv->num_kv_heads, kv, seqs);
  // the cache buffers are written: the struct's pointers are const for the
  // read-only entry points only
  return hip_status(launch_append(kv->dtype, cfg->mode, k_new, v_new, k_scale_new, v_scale_new,
                                  const_cast<void*>(kv->k), const_cast<void*>(kv->v),
                                  const_cast<uint16_t*>(kv->k_scale), const_cast<uint16_t*>(kv->v_scale),
                                  s, seqs->page_table, seqs->seq_lens, cfg->proj, meta, meta_scale,
                                  static_cast<hipStream_t>(stream)));
}

int sa_score_pages(const void* q, int32_t q_dtype, int32_t num_q_heads, const sa_kv_cache* kv,
                   const sa_seqs* seqs, const sa_select_cfg* cfg, const void* meta,
                   const uint16_t* meta_scale, float* scores, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs)) || (rc = check_cfg(cfg))) return rc;
  if ((rc = check_q(q, q_dtype, num_q_heads, kv->num_kv_heads))) return rc;
  if ((rc = check_mode_kv(cfg, kv))) return rc;
  if (!scores) return SA_ERR_INVALID_ARG;
  const Shapes s = shapes_of(num_q_heads, kv, seqs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->mode == SA_MODE_PROBE)
    return hip_status(launch_probe_score(kv->dtype, q_dtype, q, kv->k, kv->k_scale, s,
                                         seqs->page_table, seqs->seq_lens, cfg->unit_tokens,
                                         cfg->n_probe, scores, max_units_of(seqs, cfg), st));
  if (!meta || !aligned16(meta)) return SA_ERR_INVALID_ARG;
  if (cfg->mode == SA_MODE_QUEST)
    return hip_status(launch_quest_score(kv->dtype, q_dtype, q, meta, s, seqs->page_table,
                                         seqs->seq_lens, scores, st, cfg->per_head != 0));
  if (!meta_scale) return SA_ERR_INVALID_ARG;
  return hip_status(launch_sals_score(q_dtype, q, static_cast<const uint8_t*>(meta), meta_scale,
                                      cfg->proj, s, seqs->page_table, seqs->seq_lens,
                                      cfg->unit_tokens, cfg->lse_scale, scores,
                                      max_units_of(seqs, cfg), st));
}

int sa_topk_pages(const float* scores, int32_t num_kv_heads, const sa_seqs* seqs,
                  const sa_select_cfg* cfg, int32_t* sel, int32_t* num_sel, void* stream) {
  int rc;
  if ((rc = check_seqs(seqs)) || (rc = check_select(cfg))) return rc;
  if (!scores || !sel || !num_sel || num_kv_heads < 1 || num_kv_heads > 65535) return SA_ERR_INVALID_ARG;
  const Shapes s{seqs->batch, num_kv_heads, num_kv_heads, seqs->max_pages, 0};
  return hip_status(launch_topk(scores, max_units_of(seqs, cfg), s, seqs->seq_lens,
                                cfg->unit_tokens, cfg->k_compete, cfg->n_head_forced,
                                cfg->n_tail_forced, sel, num_sel, max_sel_of(seqs, cfg),
                                static_cast<hipStream_t>(stream)));
}

size_t sa_attn_heads_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_pages, int32_t max_sel) {
  if (batch < 1 || max_pages < 1 || max_pages > kUnionPages || max_sel < 1) return 0;
  if (!group_ok(num_q_heads, num_kv_heads)) return 0;
  return heads_layout(batch, num_q_heads, num_kv_heads, max_pages, max_sel).total;
}

int sa_sparse_decode_attn_heads(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                const sa_kv_cache* kv, const sa_seqs* seqs, const int32_t* sel,
                                const int32_t* num_sel, int32_t max_sel, float softmax_scale,
                                float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs))) return rc;
  if ((rc = check_q(q, q_dtype, num_q_heads, kv->num_kv_heads))) return rc;
  if (!out || !workspace || ((uintptr_t)workspace % kAlign) != 0) return SA_ERR_INVALID_ARG;
  if (!sel || !num_sel || max_sel < 1) return SA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return SA_ERR_INVALID_ARG;
  if (seqs->max_pages > kUnionPages) return SA_ERR_UNSUPPORTED;
  const HeadsLayout H = heads_layout(seqs->batch, num_q_heads, kv->num_kv_heads, seqs->max_pages, max_sel);
  if (workspace_bytes < H.total) return SA_ERR_WORKSPACE_TOO_SMALL;
  const Shapes s = shapes_of(num_q_heads, kv, seqs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* ulist = reinterpret_cast<int32_t*>(ws + H.ulist);
  int32_t* ucount = reinterpret_cast<int32_t*>(ws + H.ucount);
  rc = hip_status(launch_union(sel, num_sel, max_sel, s, seqs->seq_lens, ulist, ucount, H.umax, st));
  if (rc) return rc;
  return hip_status(launch_attention(kv->dtype, q_dtype, q, kv->k, kv->v, kv->k_scale, kv->v_scale,
                                     s, seqs->page_table, seqs->seq_lens, ulist, ucount, H.umax,
                                     H.plan, softmax_scale, reinterpret_cast<float*>(ws + H.partials),
                                     out, st, true));
}

size_t sa_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_pages, int32_t max_sel) {
  if (batch < 1 || max_pages < 1 || !group_ok(num_q_heads, num_kv_heads)) return 0;
  const AttnPlan p = plan_attention(batch, num_q_heads, num_kv_heads, max_sel > 0 ? max_sel : max_pages,
                                    max_sel <= 0);
  return align_up(p.partial_floats * sizeof(float));
}

int sa_sparse_decode_attn(const void* q, int32_t q_dtype, int32_t num_q_heads,
                          const sa_kv_cache* kv, const sa_seqs* seqs, const int32_t* sel,
                          const int32_t* num_sel, int32_t max_sel, float softmax_scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs))) return rc;
  if ((rc = check_q(q, q_dtype, num_q_heads, kv->num_kv_heads))) return rc;
  if (!out || !workspace || ((uintptr_t)workspace % kAlign) != 0) return SA_ERR_INVALID_ARG;
  if ((sel == nullptr) != (num_sel == nullptr)) return SA_ERR_INVALID_ARG;
  if (sel && max_sel < 1) return SA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return SA_ERR_INVALID_ARG;
  const int list_len = sel ? max_sel : seqs->max_pages;
  const AttnPlan plan = plan_attention(seqs->batch, num_q_heads, kv->num_kv_heads, list_len,
                                       sel == nullptr);
  if (workspace_bytes < plan.partial_floats * sizeof(float)) return SA_ERR_WORKSPACE_TOO_SMALL;
  const Shapes s = shapes_of(num_q_heads, kv, seqs);
  return hip_status(launch_attention(kv->dtype, q_dtype, q, kv->k, kv->v, kv->k_scale, kv->v_scale,
                                     s, seqs->page_table, seqs->seq_lens, sel, num_sel,
                                     sel ? max_sel : 0, plan, softmax_scale,
                                     static_cast<float*>(workspace), out,
                                     static_cast<hipStream_t>(stream)));
}

int sa_sparse_decode_attn_noalloc(const void* q, int32_t q_dtype, int32_t num_q_heads,
                                  const sa_kv_cache* kv, const sa_seqs* seqs, const int32_t* sel,
                                  const int32_t* num_sel, int32_t max_sel, float softmax_scale,
                                  float* out, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs))) return rc;
  if ((rc = check_q(q, q_dtype, num_q_heads, kv->num_kv_heads))) return rc;
  if (!out) return SA_ERR_INVALID_ARG;
  if ((sel == nullptr) != (num_sel == nullptr)) return SA_ERR_INVALID_ARG;
  if (sel && max_sel < 1) return SA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return SA_ERR_INVALID_ARG;
  const int list_len = sel ? max_sel : seqs->max_pages;
  const AttnPlan plan = plan_attention(seqs->batch, num_q_heads, kv->num_kv_heads, list_len,
                                       sel == nullptr);
  if (plan.partial_floats * sizeof(float) > kNoAllocScratchBytes) return SA_ERR_WORKSPACE_TOO_SMALL;
  float* partials = scratch_of_device();
  if (!partials) return SA_ERR_HIP;
  const Shapes s = shapes_of(num_q_heads, kv, seqs);
  return hip_status(launch_attention(kv->dtype, q_dtype, q, kv->k, kv->v, kv->k_scale, kv->v_scale,
                                     s, seqs->page_table, seqs->seq_lens, sel, num_sel,
                                     sel ? max_sel : 0, plan, softmax_scale, partials, out,
                                     static_cast<hipStream_t>(stream)));
}

size_t sa_decode_step_workspace_size(int32_t num_q_heads, const sa_kv_cache* kv,
                                     const sa_seqs* seqs, const sa_select_cfg* cfg) {
  if (check_kv(kv) || check_seqs(seqs) || check_cfg(cfg)) return 0;
  if (!group_ok(num_q_heads, kv->num_kv_heads)) return 0;
  // the larger of the layouts of the two query types the step accepts
  const size_t a = step_layout(num_q_heads, kv, seqs, cfg, SA_F32).total;
  const size_t b = step_layout(num_q_heads, kv, seqs, cfg, SA_BF16).total;
  return a > b ? a : b;
}

int sa_decode_step(const void* q, int32_t q_dtype, int32_t num_q_heads, const sa_kv_cache* kv,
                   const sa_seqs* seqs, const sa_select_cfg* cfg, const void* meta,
                   const uint16_t* meta_scale, float softmax_scale, float* out, int32_t* sel,
                   int32_t* num_sel, void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv)) || (rc = check_seqs(seqs)) || (rc = check_cfg(cfg))) return rc;
  if ((rc = check_q(q, q_dtype, num_q_heads, kv->num_kv_heads))) return rc;
  if ((rc = check_mode_kv(cfg, kv))) return rc;
  if (!out || !workspace || ((uintptr_t)workspace % kAlign) != 0) return SA_ERR_INVALID_ARG;
  if ((sel == nullptr) != (num_sel == nullptr)) return SA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return SA_ERR_INVALID_ARG;
  const StepLayout lay = step_layout(num_q_heads, kv, seqs, cfg, q_dtype);
  if (lay.per_head && seqs->max_pages > kUnionPages) return SA_ERR_UNSUPPORTED;
  if (workspace_bytes < lay.total) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (!lay.dense && cfg->mode != SA_MODE_PROBE) {
    if (!meta || !aligned16(meta)) return SA_ERR_INVALID_ARG;
    if (cfg->mode == SA_MODE_SALS && !meta_scale) return SA_ERR_INVALID_ARG;
  }
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Shapes s = shapes_of(num_q_heads, kv, seqs);
  Shapes s_lists = s;  // selection lists per sequence: the query heads with per_head
  if (cfg->per_head) s_lists.Hkv = s.Hq;
  int32_t* sel_buf = sel ? sel : reinterpret_cast<int32_t*>(ws + lay.sel);
  int32_t* num_buf = num_sel ? num_sel : reinterpret_cast<int32_t*>(ws + lay.num_sel);
  float* partials = reinterpret_cast<float*>(ws + lay.partials);

  if (lay.dense) {
    // every unit of every list is kept: selection is the identity
    if (sel) {
      rc = hip_status(launch_topk(nullptr, lay.max_units, s_lists, seqs->seq_lens, cfg->unit_tokens,
                                  cfg->k_compete, cfg->n_head_forced, cfg->n_tail_forced, sel_buf,
                                  num_buf, lay.max_sel, st));
      if (rc) return rc;
    }
    return hip_status(launch_attention(kv->dtype, q_dtype, q, kv->k, kv->v, kv->k_scale,
                                       kv->v_scale, s, seqs->page_table, seqs->seq_lens, nullptr,
                                       nullptr, 0, lay.plan, softmax_scale, partials, out, st));
  }
  float* scores = reinterpret_cast<float*>(ws + lay.scores);
  // the fused kernel's grid is the number of its workgroups the device holds at
  // once (one per CU); a build that uses scratch memory runs the separate kernels
  const int wgs = lay.fused ? resident_step_wgs(kv->dtype, q_dtype, seqs->max_pages) : 0;
  if (lay.fused && wgs >= 1) {
    StepArgs A{};
    A.q = q;
    A.k = kv->k;
    A.v = kv->v;
    A.meta = meta;
    A.pt = seqs->page_table;
    A.lens = seqs->seq_lens;
    A.B = seqs->batch;
    A.hq = num_q_heads;
    A.hkv = kv->num_kv_heads;
    A.num_pages = kv->num_pages;
    A.max_pages = seqs->max_pages;
    A.k_compete = cfg->k_compete;
    A.n_head = cfg->n_head_forced;
    A.n_tail = cfg->n_tail_forced;
    A.scale_log2 = softmax_scale * 1.4426950408889634f;
    A.scores = scores;
    A.sel = sel;
    A.num_sel = num_sel;
    A.max_sel = lay.max_sel;
    A.partials = partials;
    A.out = out;
    A.arrive = reinterpret_cast<uint32_t*>(ws + lay.arrive);
    StepPlan P = lay.splan;
    const int cap = step_wg_cap();
    P.grid = P.n_tasks < wgs ? P.n_tasks : wgs;
    if (cap > 0 && cap < P.grid) P.grid = cap;
    return hip_status(launch_quest_step(kv->dtype, q_dtype, A, P, st));
  }
  if (lay.per_head) {
    // every query head's own bound, selection and pages; the group's union read once
    rc = hip_status(launch_quest_score(kv->dtype, q_dtype, q, meta, s, seqs->page_table,
                                       seqs->seq_lens, scores, st, true));
    if (rc) return rc;
    rc = hip_status(launch_topk(scores, lay.max_units, s_lists, seqs->seq_lens, cfg->unit_tokens,
                                cfg->k_compete, cfg->n_head_forced, cfg->n_tail_forced, sel_buf,
                                num_buf, lay.max_sel, st));
    if (rc) return rc;
    char* hw = ws + lay.heads;
    int32_t* ulist = reinterpret_cast<int32_t*>(hw + lay.hl.ulist);
    int32_t* ucount = reinterpret_cast<int32_t*>(hw + lay.hl.ucount);
    rc = hip_status(launch_union(sel_buf, num_buf, lay.max_sel, s, seqs->seq_lens, ulist, ucount,
                                 lay.hl.umax, st));
    if (rc) return rc;
    return hip_status(launch_attention(kv->dtype, q_dtype, q, kv->k, kv->v, kv->k_scale,
                                       kv->v_scale, s, seqs->page_table, seqs->seq_lens, ulist,
                                       ucount, lay.hl.umax, lay.hl.plan, softmax_scale,
                                       reinterpret_cast<float*>(hw + lay.hl.partials), out, st,
                                       true));
  }
  if (cfg->mode == SA_MODE_QUEST)
    rc = hip_status(launch_quest_score(kv->dtype, q_dtype, q, meta, s, seqs->page_table,
                                       seqs->seq_lens, scores, st));
  else if (cfg->mode == SA_MODE_PROBE)
    rc = hip_status(launch_probe_score(kv->dtype, q_dtype, q, kv->k, kv->k_scale, s,
                                       seqs->page_table, seqs->seq_lens, cfg->unit_tokens,
                                       cfg->n_probe, scores, lay.max_units, st));
  else
    rc = hip_status(launch_sals_score(q_dtype, q, static_cast<const uint8_t*>(meta), meta_scale,
                                      cfg->proj, s, seqs->page_table, seqs->seq_lens,
                                      cfg->unit_tokens, cfg->lse_scale, scores, lay.max_units, st));
  if (rc) return rc;
  if (lay.post) {
    PostArgs A{};
    A.q = q;
    A.k = kv->k;
    A.v = kv->v;
    A.ks = kv->k_scale;
    A.vs = kv->v_scale;
    A.pt = seqs->page_table;
    A.lens = seqs->seq_lens;
    A.hkv = kv->num_kv_heads;
    A.num_pages = kv->num_pages;
    A.max_pages = seqs->max_pages;
    A.unit_tokens = cfg->unit_tokens;
    A.max_units = lay.max_units;
    A.k_compete = cfg->k_compete;
    A.n_head = cfg->n_head_forced;
    A.n_tail = cfg->n_tail_forced;
    A.scale_log2 = softmax_scale * kLog2e;
    A.scores = scores;
    A.sel = sel;
    A.num_sel = num_sel;
    A.max_sel = lay.max_sel;
    A.partials = partials;
    A.out = out;
    A.arrive = reinterpret_cast<uint32_t*>(ws + lay.arrive);
    PostPlan P = lay.pplan;
    const int cus = device_cus(), cap = step_wg_cap();
    P.grid = P.n_tasks < cus ? P.n_tasks : cus;
    if (cap > 0 && cap < P.grid) P.grid = cap;
    return hip_status(launch_post_score(kv->dtype, num_q_heads / kv->num_kv_heads, A, P, st));
  }
  rc = hip_status(launch_topk(scores, lay.max_units, s, seqs->seq_lens, cfg->unit_tokens,
                              cfg->k_compete, cfg->n_head_forced, cfg->n_tail_forced, sel_buf,
                              num_buf, lay.max_sel, st));
  if (rc) return rc;
  return hip_status(launch_attention(kv->dtype, q_dtype, q, kv->k, kv->v, kv->k_scale, kv->v_scale,
                                     s, seqs->page_table, seqs->seq_lens, sel_buf, num_buf,
                                     lay.max_sel, lay.plan, softmax_scale, partials, out, st));
}

int sa_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  if (!src || !aligned16(src) || bytes == 0 || bytes % 16 != 0 || !sink || sink_words < 1)
    return SA_ERR_INVALID_ARG;
  // about eight workgroups per compute unit keep enough loads in flight
  const size_t want = (size_t)device_cus() * 8;
  const int grid = (int)(sink_words < want ? sink_words : want);
  return hip_status(launch_stream_read(src, bytes, sink, grid, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
