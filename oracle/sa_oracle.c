/*
 * sa_oracle.c - plain, slow CPU oracle of query-aware sparse decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, import or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the GPU library.
 *
 * Each function follows one step of the method as the pages state it and
 * accumulates in double (decoded inputs are exact in double).  The SALS index
 * key build is the one exception: its int4 codes are an encoding that the
 * GPU must reproduce bit for bit, so it is defined in fp32 arithmetic
 * (sequential fused multiply-adds, IEEE division, round-to-nearest-even).
 *
 * Pages cited:
 *  [Quest]  "Quest 完全拆解：查询感知的页级稀疏注意力" (pinghaoyang.com.cn):
 *           page-level management; upper bound from min/max metadata and its
 *           case proof; incremental metadata update; criticality estimation,
 *           top-K filtering and approximate attention kernels; GQA section.
 *  [SALS]   "SALS长序列推理优化" (CANN learning hub): QSI steps (Q.K, dequant,
 *           block log-sum-exp, sort + top-k, append tail blocks); QSI exact
 *           top-k by stable descending sort; SFAA stages (QK, online
 *           softmax, P@V, rescale) on int8 K/V; split-row reduction.
 *  [RK]     "Day 10·2 sparse top-k 块选择" (xxmr.cn): ties go to the lower
 *           block index; the last block is always kept; no padding when
 *           there are fewer blocks than k; softmax renormalised over the
 *           selected set only.
 *  [SeqO1]  "SequenceO1" explainer (mhpn.cn): sketch attention and the
 *           two-kernel boundary; retention 100% must reproduce full attention.
 *  [RK] also: the probe signal (keys sampled evenly inside a block, the
 *           largest dot product with the query as the block's score).
 *
 * Threads: every function's outer loop runs over independent outputs (a page,
 * a (b, kv-head) list or a query head), so it is an OpenMP parallel for; no
 * value depends on the thread count.  oracle_set_threads() sets the count
 * (the Python front end starts at 1).
 *
 * Layouts (row-major):
 *   q        [B, Hq, d]              fp32 or bf16 bits
 *   K, V     [P, S, Hkv, d]          fp32, bf16 bits, or int8 codes
 *   k_scale  [P, S, Hkv]             fp16 bits (int8 caches)
 *   meta     [Hkv, P, 2, d]          KV dtype; slot 0 = per-dim max M, slot 1 = min m
 *   codes    [P, S, Hkv, rank/2]     int4 pairs, low nibble = even index
 *   scales   [P, S, Hkv]             fp16 bits
 *   page_tbl [B, max_pages]          physical page of logical page p
 * Query heads h*G .. h*G+G-1 share kv-head h (G = Hq / Hkv).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2 };

/* ---------------------------------------------------------------- decoding */
static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16 by its definition: (-1)^s * 2^(e-15) * (1 + m/1024), or
 * (-1)^s * 2^-14 * (m/1024) for e == 0. */
static double f16_value(uint16_t bits) {
  int s = bits >> 15, e = (bits >> 10) & 31, m = bits & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

/* Round a float to the nearest binary16 (ties to even) and return its bits. */
static uint16_t f16_round(float f) {
  double a = fabs((double)f);
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  if (a >= 65520.0) return sign | 0x7C00; /* rounds to infinity */
  int e2;
  frexp(a, &e2); /* a = mant * 2^e2, mant in [0.5, 1) */
  int unbiased = e2 - 1;
  double quantum = (unbiased < -14) ? ldexp(1.0, -24) : ldexp(1.0, unbiased - 10);
  double r = nearbyint(a / quantum); /* a/quantum is exact; default mode = ties to even */
  double v = r * quantum;
  if (v < ldexp(1.0, -14)) return sign | (uint16_t)nearbyint(v / ldexp(1.0, -24));
  frexp(v, &e2);
  unbiased = e2 - 1;
  int mant = (int)nearbyint((v / ldexp(1.0, unbiased) - 1.0) * 1024.0);
  return sign | (uint16_t)(((unbiased + 15) << 10) | mant);
}

static double q_value(const void *q, int q_dtype, size_t i) {
  return q_dtype == OR_F32 ? (double)((const float *)q)[i] : bf16_value(((const uint16_t *)q)[i]);
}

/* Element idx of a K or V cache; int8 codes are multiplied by the token's
 * fp16 scale (the dequantisation of the cached int8 KV [SALS, SFAA]). */
static double kv_value(const void *x, int dtype, size_t idx, const uint16_t *scale, size_t sidx) {
  switch (dtype) {
    case OR_F32: return (double)((const float *)x)[idx];
    case OR_BF16: return bf16_value(((const uint16_t *)x)[idx]);
    default: return (double)((const int8_t *)x)[idx] * f16_value(scale[sidx]);
  }
}

static size_t elem_size(int dtype) { return dtype == OR_F32 ? 4 : (dtype == OR_BF16 ? 2 : 1); }

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

/* Nonzero if a page-table entry of a referenced page (b, p < n_b) is out of range. */
static int check_pages(const int32_t *page_table, const int32_t *seq_lens, int B, int max_pages,
                       int S, int num_pages) {
  for (int b = 0; b < B; ++b) {
    int n = ceil_div(seq_lens[b], S);
    for (int p = 0; p < n && p < max_pages; ++p) {
      int pp = page_table[(size_t)b * max_pages + p];
      if (pp < 0 || pp >= num_pages) return 1;
    }
  }
  return 0;
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n < 1 ? 1 : n);
#else
  (void)n;
#endif
}

/* -------------------------------------------------- page metadata (min/max) */
/*
 * [Quest] incremental update: inserting key k into a page sets
 * M_i <- max(M_i, k_i) and m_i <- min(m_i, k_i).  Folding that update over the
 * page's valid tokens in slot order gives the per-dimension max and min.  The
 * chosen element is copied bit for bit, so the metadata stays in the KV dtype
 * (exact; an earlier equal value is kept on ties).
 */
int oracle_quest_meta(const void *k, int dtype, int num_pages, int S, int hkv, int d,
                      const int32_t *page_table, const int32_t *seq_lens, int B, int max_pages,
                      void *meta) {
  if (dtype == OR_I8) return -1;
  if (check_pages(page_table, seq_lens, B, max_pages, S, num_pages)) return -2;
  size_t es = elem_size(dtype);
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int b = 0; b < B; ++b) {
    for (int p = 0; p < max_pages; ++p) {
      int L = seq_lens[b];
      if (p >= ceil_div(L, S)) continue;
      int pp = page_table[(size_t)b * max_pages + p];
      int valid = L - p * S < S ? L - p * S : S;
      for (int h = 0; h < hkv; ++h) {
        for (int i = 0; i < d; ++i) {
          size_t i0 = (((size_t)pp * S + 0) * hkv + h) * d + i;
          double mx = kv_value(k, dtype, i0, NULL, 0), mn = mx;
          size_t at_mx = i0, at_mn = i0;
          for (int s = 1; s < valid; ++s) {
            size_t is = (((size_t)pp * S + s) * hkv + h) * d + i;
            double x = kv_value(k, dtype, is, NULL, 0);
            if (x > mx) { mx = x; at_mx = is; }
            if (x < mn) { mn = x; at_mn = is; }
          }
          uint8_t *dst = (uint8_t *)meta;
          size_t oM = (((size_t)h * num_pages + pp) * 2 + 0) * d + i;
          size_t om = (((size_t)h * num_pages + pp) * 2 + 1) * d + i;
          memcpy(dst + oM * es, (const uint8_t *)k + at_mx * es, es);
          memcpy(dst + om * es, (const uint8_t *)k + at_mn * es, es);
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------- Quest page scores */
/*
 * [Quest] criticality estimation: score = sum_i max(q_i * m_i, q_i * M_i),
 * an upper bound of q.k for every key k of the page (case proof on the sign of
 * q_i).  [Quest] GQA section: one selection is shared by the query heads of a
 * group; the group score is the max over its heads of the per-head bound, so
 * that for every head it still bounds that head's largest true dot product.
 * abs_scale (optional) = max over the group of sum_i |q_i| * max(|m_i|, |M_i|):
 * the magnitude the rounding error of a float evaluation is relative to.
 * Pages p >= n_b get -inf.
 */
void oracle_quest_scores(const void *q, int q_dtype, int hq, const void *meta, int dtype, int hkv,
                         int num_pages, int d, int S, const int32_t *page_table,
                         const int32_t *seq_lens, int B, int max_pages, double *scores,
                         double *abs_scale) {
  int G = hq / hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < hkv; ++h) {
      int n = ceil_div(seq_lens[b], S);
      for (int p = 0; p < max_pages; ++p) {
        size_t o = ((size_t)b * hkv + h) * max_pages + p;
        if (p >= n) {
          scores[o] = -INFINITY;
          if (abs_scale) abs_scale[o] = 0.0;
          continue;
        }
        int pp = page_table[(size_t)b * max_pages + p];
        double best = -INFINITY, best_a = 0.0;
        for (int g = 0; g < G; ++g) {
          size_t qo = ((size_t)b * hq + (size_t)h * G + g) * d;
          double s = 0.0, a = 0.0;
          for (int i = 0; i < d; ++i) {
            double qi = q_value(q, q_dtype, qo + i);
            double Mi = kv_value(meta, dtype, (((size_t)h * num_pages + pp) * 2 + 0) * d + i, NULL, 0);
            double mi = kv_value(meta, dtype, (((size_t)h * num_pages + pp) * 2 + 1) * d + i, NULL, 0);
            double u1 = qi * mi, u2 = qi * Mi;
            s += u1 > u2 ? u1 : u2;
            a += fabs(qi) * (fabs(Mi) > fabs(mi) ? fabs(Mi) : fabs(mi));
          }
          if (s > best) best = s;
          if (a > best_a) best_a = a;
        }
        scores[o] = best;
        if (abs_scale) abs_scale[o] = best_a;
      }
    }
  }
}

/* -------------------------------------------------------- SALS index key */
/*
 * [SALS] low-rank preprocessing + int4 index key, [SeqO1] sketch K*P.
 * Per (token, kv-head), all in fp32:
 *   khat_i = key value (int8 caches: (float)code * (float)scale, exact);
 *   kp_j   = fmaf chain over i = 0..d-1 from 0: kp_j = fmaf(khat_i, P[i][j], kp_j);
 *   scale  = fp16 round-to-nearest-even of (max_j |kp_j|) / 7   (IEEE fp32 division);
 *   c_j    = clamp(rintf(kp_j / scale), -7, 7), all 0 when scale == 0;
 *   two codes per byte, low nibble = even j.
 * Slots past the sequence end in a referenced page are written as zeros.
 */
int oracle_sals_index(const void *k, int dtype, const uint16_t *k_scale, int num_pages, int S,
                      int hkv, int d, const int32_t *page_table, const int32_t *seq_lens, int B,
                      int max_pages, const float *proj, int rank, uint8_t *codes,
                      uint16_t *scales) {
  if (rank % 2 != 0 || rank > 64 || d > 1024) return -1;
  if (check_pages(page_table, seq_lens, B, max_pages, S, num_pages)) return -2;
  int nb = rank / 2;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int b = 0; b < B; ++b) {
    for (int p = 0; p < max_pages; ++p) {
      float khat[1024], kp[64];
      int L = seq_lens[b];
      if (p >= ceil_div(L, S)) continue;
      int pp = page_table[(size_t)b * max_pages + p];
      for (int s = 0; s < S; ++s) {
        for (int h = 0; h < hkv; ++h) {
          size_t row = ((size_t)pp * S + s) * hkv + h;
          uint8_t *crow = codes + row * nb;
          if (p * S + s >= L) {
            memset(crow, 0, (size_t)nb);
            scales[row] = 0;
            continue;
          }
          for (int i = 0; i < d; ++i) {
            size_t idx = row * d + i;
            if (dtype == OR_F32)
              khat[i] = ((const float *)k)[idx];
            else if (dtype == OR_BF16)
              khat[i] = (float)bf16_value(((const uint16_t *)k)[idx]);
            else
              khat[i] = (float)((const int8_t *)k)[idx] * (float)f16_value(k_scale[row]);
          }
          float amax = 0.0f;
          for (int j = 0; j < rank; ++j) {
            float acc = 0.0f;
            for (int i = 0; i < d; ++i) acc = fmaf(khat[i], proj[(size_t)i * rank + j], acc);
            kp[j] = acc;
            if (fabsf(acc) > amax) amax = fabsf(acc);
          }
          uint16_t sh = f16_round(amax / 7.0f);
          float sf = (float)f16_value(sh);
          scales[row] = sh;
          for (int m = 0; m < nb; ++m) {
            int c[2];
            for (int e = 0; e < 2; ++e) {
              float v = 0.0f;
              if (sf != 0.0f) {
                v = rintf(kp[2 * m + e] / sf);
                if (v > 7.0f) v = 7.0f;
                if (v < -7.0f) v = -7.0f;
              }
              c[e] = (int)v;
            }
            crow[m] = (uint8_t)((c[0] & 0xF) | ((c[1] & 0xF) << 4));
          }
        }
      }
    }
  }
  return 0;
}

/* ----------------------------------------------------------- SALS scores */
static int nibble(const uint8_t *row, int j) {
  int v = (j & 1) ? (row[j >> 1] >> 4) : (row[j >> 1] & 0xF);
  return v >= 8 ? v - 16 : v;
}

/* log sum exp over n values, max-subtracted. */
static double log_sum_exp(const double *z, int n) {
  double m = -INFINITY;
  for (int t = 0; t < n; ++t)
    if (z[t] > m) m = z[t];
  double s = 0.0;
  for (int t = 0; t < n; ++t) s += exp(z[t] - m);
  return m + log(s);
}

/*
 * Shared body of the SALS block scorer.  For (b, kv-head h):
 *   qbar = mean of the group's query heads  [SALS: the index query is the
 *          group-mean of q];
 *   qt   = qbar * P (rank values);
 *   per token t: s_t = sum_j qt_j * key_lr(t, j)  [SALS steps 1-2: Q.K, dequant];
 *   per unit (block of unit_tokens tokens) u: LSE_u = log sum over valid t in u of
 *        exp(tau * s_t)  [SALS step 3, block log-sum-exp].
 * key_lr is the dequantised low-rank key: scale_t * c_tj for the int4 index,
 * or a float array for the unquantised generalisation.
 */
typedef double (*lowrank_key_fn)(const void *ctx, size_t row, int j);

struct codes_ctx { const uint8_t *codes; const uint16_t *scales; int nb; };
static double key_from_codes(const void *c, size_t row, int j) {
  const struct codes_ctx *x = (const struct codes_ctx *)c;
  return f16_value(x->scales[row]) * (double)nibble(x->codes + row * x->nb, j);
}
struct float_ctx { const float *keys; int rank; };
static double key_from_floats(const void *c, size_t row, int j) {
  const struct float_ctx *x = (const struct float_ctx *)c;
  return (double)x->keys[row * x->rank + j];
}

static void sals_scores_body(const void *q, int q_dtype, int hq, lowrank_key_fn key, const void *ctx,
                             int hkv, int S, int rank, const float *proj, int d,
                             const int32_t *page_table, const int32_t *seq_lens, int B,
                             int max_pages, int unit_tokens, double tau, double *scores,
                             double *abs_scale) {
  int G = hq / hkv;
  int max_units = ceil_div(max_pages * S, unit_tokens);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < hkv; ++h) {
      double *qbar = (double *)malloc(sizeof(double) * (size_t)d);
      double *qt = (double *)malloc(sizeof(double) * (size_t)rank);
      double *z = (double *)malloc(sizeof(double) * (size_t)unit_tokens);
      int L = seq_lens[b];
      int nu = ceil_div(L, unit_tokens);
      for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int g = 0; g < G; ++g) s += q_value(q, q_dtype, ((size_t)b * hq + (size_t)h * G + g) * d + i);
        qbar[i] = s / G;
      }
      for (int j = 0; j < rank; ++j) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += qbar[i] * (double)proj[(size_t)i * rank + j];
        qt[j] = s;
      }
      for (int u = 0; u < max_units; ++u) {
        size_t o = ((size_t)b * hkv + h) * max_units + u;
        if (u >= nu) {
          scores[o] = -INFINITY;
          if (abs_scale) abs_scale[o] = 0.0;
          continue;
        }
        int t0 = u * unit_tokens, t1 = t0 + unit_tokens < L ? t0 + unit_tokens : L;
        double amax = 0.0;
        for (int t = t0; t < t1; ++t) {
          int pp = page_table[(size_t)b * max_pages + t / S];
          size_t row = ((size_t)pp * S + (t % S)) * hkv + h;
          double s = 0.0, a = 0.0;
          for (int j = 0; j < rank; ++j) {
            double kj = key(ctx, row, j);
            s += qt[j] * kj;
            a += fabs(qt[j] * kj);
          }
          z[t - t0] = tau * s;
          if (tau * a > amax) amax = tau * a;
        }
        scores[o] = log_sum_exp(z, t1 - t0);
        if (abs_scale) abs_scale[o] = amax + 1.0;
      }
      free(qbar);
      free(qt);
      free(z);
    }
  }
}

/* SALS block scores from the int4 index key (codes + fp16 scales). */
void oracle_sals_scores(const void *q, int q_dtype, int hq, const uint8_t *codes,
                        const uint16_t *scales, int hkv, int S, int rank, const float *proj, int d,
                        const int32_t *page_table, const int32_t *seq_lens, int B, int max_pages,
                        int unit_tokens, double tau, double *scores, double *abs_scale) {
  struct codes_ctx c = {codes, scales, rank / 2};
  sals_scores_body(q, q_dtype, hq, key_from_codes, &c, hkv, S, rank, proj, d, page_table, seq_lens,
                   B, max_pages, unit_tokens, tau, scores, abs_scale);
}

/* Same scorer on unquantised low-rank keys [P, S, Hkv, rank] (fp32). */
void oracle_sals_scores_float(const void *q, int q_dtype, int hq, const float *keys, int hkv, int S,
                              int rank, const float *proj, int d, const int32_t *page_table,
                              const int32_t *seq_lens, int B, int max_pages, int unit_tokens,
                              double tau, double *scores) {
  struct float_ctx c = {keys, rank};
  sals_scores_body(q, q_dtype, hq, key_from_floats, &c, hkv, S, rank, proj, d, page_table,
                   seq_lens, B, max_pages, unit_tokens, tau, scores, NULL);
}

/* ---------------------------------------------------------- selection */
struct unit_score { double s; int u; };

/* score descending, then index ascending [SALS stable descending sort; RK tie rule] */
static int by_score_then_index(const void *a, const void *b) {
  const struct unit_score *x = (const struct unit_score *)a, *y = (const struct unit_score *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->u > y->u) - (x->u < y->u);
}

/*
 * Per (b, kv-head): n units (pages, or blocks of unit_tokens tokens).  The
 * first n_head and last n_tail units are always kept ([Quest]/[RK]: sink page
 * and recent page; [SALS]: fixed tail blocks appended).  If n <= n_head +
 * n_tail + k every unit is kept (no padding, [RK]); otherwise the k best
 * middle units by (score desc, index asc) are kept.  The kept units are
 * listed in ascending order and expanded to their logical pages (clipped to
 * the sequence).  Unused entries of sel are -1.  Returns -1 if a list would
 * exceed max_sel.
 */
int oracle_select(const double *scores, int B, int hkv, int max_units, const int32_t *seq_lens,
                  int S, int unit_tokens, int k, int n_head, int n_tail, int max_sel, int32_t *sel,
                  int32_t *num_sel) {
  int upu = unit_tokens / S;
  int rc = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(min : rc)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < hkv; ++h) {
      struct unit_score *buf = (struct unit_score *)malloc(sizeof(struct unit_score) * (size_t)(max_units + 1));
      unsigned char *keep = (unsigned char *)malloc((size_t)max_units + 1);
      int L = seq_lens[b];
      int n = ceil_div(L, unit_tokens);
      int np = ceil_div(L, S);
      const double *sc = scores + ((size_t)b * hkv + h) * max_units;
      memset(keep, 0, (size_t)max_units + 1);
      if (n <= n_head + n_tail + k) {
        for (int u = 0; u < n; ++u) keep[u] = 1;
      } else {
        for (int u = 0; u < n_head; ++u) keep[u] = 1;
        for (int u = n - n_tail; u < n; ++u) keep[u] = 1;
        int m = 0;
        for (int u = n_head; u < n - n_tail; ++u) {
          buf[m].s = sc[u];
          buf[m].u = u;
          ++m;
        }
        qsort(buf, (size_t)m, sizeof(struct unit_score), by_score_then_index);
        for (int r = 0; r < k; ++r) keep[buf[r].u] = 1;
      }
      int32_t *out = sel + ((size_t)b * hkv + h) * max_sel;
      int cnt = 0;
      for (int u = 0; u < n; ++u) {
        if (!keep[u]) continue;
        for (int p = u * upu; p < (u + 1) * upu && p < np; ++p) {
          if (cnt >= max_sel) { rc = -1; break; }
          out[cnt++] = p;
        }
      }
      for (int r = cnt; r < max_sel; ++r) out[r] = -1;
      num_sel[(size_t)b * hkv + h] = cnt;
      free(buf);
      free(keep);
    }
  }
  return rc;
}

/* ---------------------------------------------------------- attention */
/*
 * Exact softmax attention of one query head over the valid tokens of the
 * given logical pages ([Quest] approximate attention over the selected pages;
 * [SALS] SFAA on dequantised int8 K/V; [RK] softmax renormalised over the
 * selected set only):
 *   z_t = tau * sum_i q_i k_ti,  w_t = exp(z_t - max z),  out = sum_t w_t v_t / sum_t w_t.
 * sel == NULL attends to every page [0, n_b) (dense attention, [SeqO1]: 100%
 * retention reproduces full attention).  rows (optional) lists flattened
 * (b * Hq + head) indices; the output is then [nrows, d], else [B, Hq, d].
 * An empty token set yields zeros.
 */
void oracle_attention(const void *q, int q_dtype, int hq, const void *k, const void *v, int dtype,
                      const uint16_t *k_scale, const uint16_t *v_scale, int hkv, int d, int S,
                      const int32_t *page_table, const int32_t *seq_lens, int B, int max_pages,
                      const int32_t *sel, const int32_t *num_sel, int max_sel, double tau,
                      const int32_t *rows, int nrows, float *out) {
  int G = hq / hkv;
  int total = rows ? nrows : B * hq;
  size_t cap = (size_t)max_pages * S;
#pragma omp parallel
  {
  double *z = (double *)malloc(sizeof(double) * (cap ? cap : 1));
  size_t *tok = (size_t *)malloc(sizeof(size_t) * (cap ? cap : 1));
  double *acc = (double *)malloc(sizeof(double) * (size_t)d);
  double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
  for (int r = 0; r < total; ++r) {
    int flat = rows ? rows[r] : r;
    int b = flat / hq, head = flat % hq, h = head / G;
    for (int i = 0; i < d; ++i) qrow[i] = q_value(q, q_dtype, ((size_t)b * hq + head) * d + i);
    int L = seq_lens[b];
    int np = ceil_div(L, S);
    int cnt = sel ? num_sel[(size_t)b * hkv + h] : np;
    const int32_t *lst = sel ? sel + ((size_t)b * hkv + h) * max_sel : NULL;
    size_t nt = 0;
    for (int c = 0; c < cnt; ++c) {
      int p = lst ? lst[c] : c;
      int pp = page_table[(size_t)b * max_pages + p];
      for (int s = 0; s < S; ++s) {
        if (p * S + s >= L) break;
        size_t row = ((size_t)pp * S + s) * hkv + h;
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += qrow[i] * kv_value(k, dtype, row * d + i, k_scale, row);
        z[nt] = tau * dot;
        tok[nt] = row;
        ++nt;
      }
    }
    float *o = out + (size_t)r * d;
    if (nt == 0) {
      for (int i = 0; i < d; ++i) o[i] = 0.0f;
      continue;
    }
    double m = -INFINITY;
    for (size_t t = 0; t < nt; ++t)
      if (z[t] > m) m = z[t];
    double l = 0.0;
    for (int i = 0; i < d; ++i) acc[i] = 0.0;
    for (size_t t = 0; t < nt; ++t) {
      double w = exp(z[t] - m);
      l += w;
      for (int i = 0; i < d; ++i) acc[i] += w * kv_value(v, dtype, tok[t] * d + i, v_scale, tok[t]);
    }
    for (int i = 0; i < d; ++i) o[i] = (float)(acc[i] / l);
  }
  free(z);
  free(tok);
  free(acc);
  free(qrow);
  }
}

/* ------------------------------------------------- probe-sampling scores
 * [RK] §1-§2 (the probe signal of the block selector): a block's potential
 * attention score is the largest dot product of the query with a few keys
 * taken evenly inside the block, so a needle in the middle of an otherwise
 * dull block is not missed, at a cost of n_probe rows per block.
 * Block u of sequence b covers positions [u*U, min((u+1)*U, L)); with len its
 * token count and step = max(1, len / n_probe) (integer division), the probed
 * positions are u*U, u*U + step, u*U + 2*step, ... below the block end.
 * score = max over the probed tokens t and over the group's query heads g of
 * q_g . k_t (unscaled; GQA groups share one selection, as for Quest).  Blocks
 * past the sequence get -inf.  abs_scale = max over the same (t, g) of
 * sum_i |q_gi k_ti| (the magnitude the fp32 sums are judged against).
 */
void oracle_probe_scores(const void *q, int q_dtype, int hq, const void *k, int dtype,
                         const uint16_t *k_scale, int hkv, int S, int d, const int32_t *page_table,
                         const int32_t *seq_lens, int B, int max_pages, int unit_tokens, int n_probe,
                         double *scores, double *abs_scale) {
  int G = hq / hkv;
  int max_units = ceil_div(max_pages * S, unit_tokens);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < hkv; ++h) {
      int L = seq_lens[b];
      int nu = ceil_div(L, unit_tokens);
      for (int u = 0; u < max_units; ++u) {
        size_t o = ((size_t)b * hkv + h) * max_units + u;
        if (u >= nu) {
          scores[o] = -INFINITY;
          if (abs_scale) abs_scale[o] = 0.0;
          continue;
        }
        int t0 = u * unit_tokens, t1 = t0 + unit_tokens < L ? t0 + unit_tokens : L;
        int step = (t1 - t0) / n_probe;
        if (step < 1) step = 1;
        double best = -INFINITY, amax = 0.0;
        for (int t = t0; t < t1; t += step) {
          int pp = page_table[(size_t)b * max_pages + t / S];
          size_t row = ((size_t)pp * S + (t % S)) * hkv + h;
          for (int g = 0; g < G; ++g) {
            double dot = 0.0, a = 0.0;
            for (int i = 0; i < d; ++i) {
              double x = q_value(q, q_dtype, ((size_t)b * hq + (size_t)h * G + g) * d + i) *
                         kv_value(k, dtype, row * d + i, k_scale, row);
              dot += x;
              a += fabs(x);
            }
            if (dot > best) best = dot;
            if (a > amax) amax = a;
          }
        }
        scores[o] = best;
        if (abs_scale) abs_scale[o] = amax;
      }
    }
  }
}

int oracle_abi_version(void) { return 1; }
