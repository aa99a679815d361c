/*
 * CPU oracle for dynamic block-sparse causal prefill attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * It follows the three stages of the FlashPrefill summary page (paperlayer.ai,
 * "FlashPrefill: Instantaneous Pattern Discovery and Thresholding for
 * Ultra-Fast Long-Context Prefilling", Appendix B "Detailed Implementation"
 * and section 3 "Method"), step by step, in plain loops with double precision
 * accumulation:
 *
 *   pool    mean of the B tokens of every block (section 3, "average-pooled
 *           key blocks"; Appendix B, "pre-pools key blocks"); queries are
 *           pooled the same way (the block-level reading of the cross-query
 *           averaging in section 3, see the reading notes below);
 *   score   S[h,I,J] = c * Qbar[h,I] . Kbar[g(h),J] for causally valid J <= I,
 *           then a softmax over J <= I (Appendix B, "causally valid pooled key
 *           blocks" and "global normalization");
 *   mask    keep J when P >= gamma * max_J P (section 3, "Max-based Dynamic
 *           Thresholding"; Appendix B, blocks whose scores "reach alpha times
 *           the per-query-block maximum"), OR the sink blocks and the local
 *           window (Appendix A), AND causal; compressed to ascending index
 *           lists (Appendix B, "active-block indices are compressed");
 *   attn    for every query token, exact softmax attention over the tokens of
 *           its kept key blocks that are causally visible (Appendix B,
 *           "Block Sparse Attention ... causal masking where required ...
 *           final normalization").  The oracle takes the plain definition
 *           (two passes: max, then normalised sum), not the online update:
 *           the online softmax reaches the same value up to rounding order.
 *
 * Readings where the page is silent (each also listed in the design notes):
 *   - c = sm_scale, default 1/sqrt(d), the attention scale;
 *   - ties at the threshold are kept (>=); gamma = 0 keeps every causal block;
 *   - the row maximum is taken over every causal J, forced blocks included;
 *   - GQA: q head h reads kv head h / (hq / hkv);
 *   - a ragged last block (seq not a multiple of B) pools over its valid
 *     tokens only; keys >= seq do not exist;
 *   - fp8 inputs are OCP e4m3fn codes times a per-head fp32 scale;
 *     pooled values are means of the dequantised values.
 *
 * Storage dtypes: 0 = float32, 1 = bfloat16 bits, 2 = e4m3fn codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_FP8 2

/* bfloat16 is the top half of an IEEE binary32 word. */
static double dec_bf16(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP e4m3fn by its definition: sign, 4-bit exponent with bias 7, 3-bit
 * mantissa; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no inf. */
double oracle_decode_e4m3fn(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

double oracle_decode_bf16(uint16_t b) { return dec_bf16(b); }

static double e4m3_table[256];
static int e4m3_ready = 0;

static void init_tables(void) {
  if (!e4m3_ready) {
    for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_decode_e4m3fn((uint8_t)c);
    e4m3_ready = 1;
  }
}

/* element idx of a storage tensor, times the head scale (1 unless fp8) */
static inline double load(const void *x, int dtype, size_t idx) {
  switch (dtype) {
    case OR_F32: return (double)((const float *)x)[idx];
    case OR_BF16: return dec_bf16(((const uint16_t *)x)[idx]);
    default: return e4m3_table[((const uint8_t *)x)[idx]];
  }
}

static int nthreads_used = 1;
int oracle_threads(void) { return nthreads_used; }

/* Block mean pooling.  x: [heads][seq][d]; scales: per-head (fp8) or NULL.
 * out: [heads][nb][d], nb = ceil(seq / block). */
int oracle_pool(int heads, int seq, int d, int block, int dtype, const void *x,
                const float *scales, double *out) {
  init_tables();
  int nb = (seq + block - 1) / block;
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < heads; ++h)
    for (int I = 0; I < nb; ++I) {
      double s = scales ? (double)scales[h] : 1.0;
      int t0 = I * block, t1 = t0 + block < seq ? t0 + block : seq;
      double *o = out + ((size_t)h * nb + I) * d;
      for (int e = 0; e < d; ++e) o[e] = 0.0;
      for (int t = t0; t < t1; ++t)
        for (int e = 0; e < d; ++e) o[e] += load(x, dtype, ((size_t)h * seq + t) * d + e);
      for (int e = 0; e < d; ++e) o[e] = o[e] * s / (double)(t1 - t0);
    }
#ifdef _OPENMP
  nthreads_used = omp_get_max_threads();
#endif
  return 0;
}

/* Block scores and their per-row softmax over causally valid key blocks.
 * qbar: [hq][nb][d], kbar: [hkv][nb][d]; S and P: [hq][nb][nb]; entries with
 * J > I are 0 in both (S is optional, may be NULL). */
int oracle_score(int hq, int hkv, int nb, int d, const double *qbar, const double *kbar,
                 double c, double *S, double *P) {
  int grp = hq / hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int h = 0; h < hq; ++h)
    for (int I = 0; I < nb; ++I) {
      int g = h / grp;
      const double *qi = qbar + ((size_t)h * nb + I) * d;
      double *prow = P + ((size_t)h * nb + I) * nb;
      double m = -INFINITY, l = 0.0;
      for (int J = 0; J < nb; ++J) prow[J] = 0.0;
      for (int J = 0; J <= I; ++J) {
        const double *kj = kbar + ((size_t)g * nb + J) * d;
        double s = 0.0;
        for (int e = 0; e < d; ++e) s += qi[e] * kj[e];
        s *= c;
        prow[J] = s; /* logits first */
        if (s > m) m = s;
      }
      if (S) {
        double *srow = S + ((size_t)h * nb + I) * nb;
        for (int J = 0; J < nb; ++J) srow[J] = J <= I ? prow[J] : 0.0;
      }
      for (int J = 0; J <= I; ++J) l += exp(prow[J] - m);
      for (int J = 0; J <= I; ++J) prow[J] = exp(prow[J] - m) / l;
    }
#ifdef _OPENMP
  nthreads_used = omp_get_max_threads();
#endif
  return 0;
}

/* Per-query block approximation (section 3 "Instantaneous Pattern Discovery":
 * pooled key blocks stand in for their tokens, and the block-level
 * significance is the average over the queries of a block; "Block
 * Approximation for Kernel Optimization": the result lives on the
 * (L/B) x (L/B) grid).  For every query token i of block I and every
 * causally valid key block J <= I:
 *   s_iJ = c * q_i . kbar_J,   p_iJ = exp(s_iJ) / sum_{J' <= I} exp(s_iJ')
 *   P[I][J] = mean over the valid tokens i of block I of p_iJ,  0 for J > I.
 * q: [hq][seq][d] storage values (fp8 codes times q_scale[h]); kbar: pooled
 * keys [hkv][nb][d] from oracle_pool.  rows: NULL for every (h, I), output
 * [hq][nb][nb]; else nrow flat row ids h*nb + I, output [nrow][nb]. */
int oracle_score_arith(int hq, int hkv, int seq, int d, int block, int dtype, const void *q,
                       const float *q_scale, const double *kbar, double c, long nrow,
                       const long *rows, double *P) {
  init_tables();
  int nb = (seq + block - 1) / block, grp = hq / hkv;
  long n = rows ? nrow : (long)hq * nb;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)nb);
    double *qi = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
    for (long t = 0; t < n; ++t) {
      long r = rows ? rows[t] : t;
      int h = (int)(r / nb), I = (int)(r % nb), g = h / grp;
      double *prow = P + (size_t)t * nb;
      double qs = q_scale ? (double)q_scale[h] : 1.0;
      for (int J = 0; J < nb; ++J) prow[J] = 0.0;
      int i0 = I * block, i1 = i0 + block < seq ? i0 + block : seq;
      for (int i = i0; i < i1; ++i) {
        for (int e = 0; e < d; ++e) qi[e] = load(q, dtype, ((size_t)h * seq + i) * d + e) * qs;
        double m = -INFINITY, z = 0.0;
        for (int J = 0; J <= I; ++J) {
          const double *kj = kbar + ((size_t)g * nb + J) * d;
          double acc = 0.0;
          for (int e = 0; e < d; ++e) acc += qi[e] * kj[e];
          s[J] = c * acc;
          if (s[J] > m) m = s[J];
        }
        for (int J = 0; J <= I; ++J) z += exp(s[J] - m);
        for (int J = 0; J <= I; ++J) prow[J] += exp(s[J] - m) / z;
      }
      for (int J = 0; J <= I; ++J) prow[J] /= (double)(i1 - i0);
    }
    free(s);
    free(qi);
  }
#ifdef _OPENMP
  nthreads_used = omp_get_max_threads();
#endif
  return 0;
}

/* Max-based dynamic threshold plus structural blocks, then compaction.
 * P: [hq][nb][nb] (only J <= I is read) or NULL when user_mask is given;
 * user_mask: optional [hq][nb][nb], replaces the threshold and the forced
 * blocks, still ANDed with causal.
 * Outputs mask [hq][nb][nb] (0/1), idx [hq][nb][nb] (ascending J, first cnt
 * valid, the rest set to -1) and cnt [hq][nb]. */
int oracle_mask(int hq, int nb, const double *P, const uint8_t *user_mask, double gamma,
                int sink_blocks, int local_blocks, uint8_t *mask, int32_t *idx,
                int32_t *cnt) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < hq; ++h)
    for (int I = 0; I < nb; ++I) {
      size_t row = (size_t)h * nb + I;
      uint8_t *mrow = mask + row * nb;
      int32_t *irow = idx + row * nb;
      double pmax = -INFINITY;
      if (!user_mask)
        for (int J = 0; J <= I; ++J)
          if (P[row * nb + J] > pmax) pmax = P[row * nb + J];
      int n = 0;
      for (int J = 0; J < nb; ++J) {
        int keep;
        if (J > I)
          keep = 0;
        else if (user_mask)
          keep = user_mask[row * nb + J] != 0;
        else
          keep = P[row * nb + J] >= gamma * pmax || J < sink_blocks || I - J < local_blocks;
        mrow[J] = (uint8_t)keep;
        if (keep) irow[n++] = J;
      }
      for (int J = n; J < nb; ++J) irow[J] = -1;
      cnt[row] = n;
    }
  return 0;
}

/* Block-sparse causal attention for a list of query tokens.
 * q: [hq][seq][d], k, v: [hkv][seq][d] (storage dtype), per-head scales for
 * fp8 (NULL otherwise).  mask: [hq][nb][nb] kept blocks (J > I ignored).
 * rows: n flat query ids h*seq + i (NULL = all hq*seq in order).
 * out: [n][d]; lse: [n] natural-log sum of exp of the scaled logits over the
 * kept causal keys (-inf and out = 0 for an empty set). */
int oracle_attn(int hq, int hkv, int seq, int d, int block, int dtype, const void *q,
                const void *k, const void *v, const float *q_scale, const float *k_scale,
                const float *v_scale, double sm_scale, const uint8_t *mask, int64_t n,
                const int64_t *rows, double *out, double *lse) {
  init_tables();
  int nb = (seq + block - 1) / block;
  int grp = hq / hkv;
  if (!rows) n = (int64_t)hq * seq;
#pragma omp parallel
  {
    double *logit = (double *)malloc(sizeof(double) * (size_t)seq);
    double *qv = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
      int64_t flat = rows ? rows[r] : r;
      int h = (int)(flat / seq), i = (int)(flat % seq);
      int g = h / grp, I = i / block;
      double qs = q_scale ? (double)q_scale[h] : 1.0;
      double ks = k_scale ? (double)k_scale[g] : 1.0;
      double vs = v_scale ? (double)v_scale[g] : 1.0;
      const uint8_t *mrow = mask + ((size_t)h * nb + I) * nb;
      for (int e = 0; e < d; ++e) qv[e] = load(q, dtype, ((size_t)h * seq + i) * d + e) * qs;
      /* pass 1: logits of the visible keys and their maximum */
      double m = -INFINITY;
      for (int j = 0; j <= i; ++j) {
        if (!mrow[j / block]) continue;
        double s = 0.0;
        for (int e = 0; e < d; ++e) s += qv[e] * (load(k, dtype, ((size_t)g * seq + j) * d + e) * ks);
        s *= sm_scale;
        logit[j] = s;
        if (s > m) m = s;
      }
      double *o = out + (size_t)r * d;
      for (int e = 0; e < d; ++e) o[e] = 0.0;
      if (m == -INFINITY) {
        lse[r] = -INFINITY;
        continue;
      }
      /* pass 2: normaliser, then the probability-weighted sum of V */
      double l = 0.0;
      for (int j = 0; j <= i; ++j)
        if (mrow[j / block]) l += exp(logit[j] - m);
      for (int j = 0; j <= i; ++j) {
        if (!mrow[j / block]) continue;
        double p = exp(logit[j] - m) / l;
        for (int e = 0; e < d; ++e) o[e] += p * (load(v, dtype, ((size_t)g * seq + j) * d + e) * vs);
      }
      lse[r] = m + log(l);
    }
    free(logit);
    free(qv);
  }
#ifdef _OPENMP
  nthreads_used = omp_get_max_threads();
#endif
  (void)nb;
  return 0;
}

/* ---------------------------------------------------------------- rescue
 * Radius-based rescue branch (thelatestinai page, RBS-Attention abstract: a
 * centroid base branch plus a rescue branch built on the maximum key-block
 * radius, each thresholded on its own, masks combined).  The page gives no
 * formula; the reading taken here:
 *   radius  r[g][J] = max over the valid keys k of block J of ||k - Kbar_J||
 *   rescue  R[h][I][J] = c * (Qbar_I . Kbar_J + ||Qbar_I|| * r[g][J]),
 *           an upper bound on c * Qbar_I . k for every key k of block J
 *           (Cauchy-Schwarz), row-softmaxed over J <= I like the base score;
 *   mask    keep = causal AND (base keep OR rescue keep OR forced), each
 *           branch with its own max-based threshold factor. */

/* k: [hkv][seq][d] storage values (fp8 codes times k_scale[g]); kbar from
 * oracle_pool on the same keys.  r: [hkv][nb]. */
int oracle_key_radius(int hkv, int seq, int d, int block, int dtype, const void *k,
                      const float *k_scale, const double *kbar, double *r) {
  init_tables();
  int nb = (seq + block - 1) / block;
#pragma omp parallel for collapse(2) schedule(static)
  for (int g = 0; g < hkv; ++g)
    for (int J = 0; J < nb; ++J) {
      double s = k_scale ? (double)k_scale[g] : 1.0, best = 0.0;
      const double *m = kbar + ((size_t)g * nb + J) * d;
      int t1 = (J + 1) * block < seq ? (J + 1) * block : seq;
      for (int t = J * block; t < t1; ++t) {
        double d2 = 0.0;
        for (int e = 0; e < d; ++e) {
          double x = load(k, dtype, ((size_t)g * seq + t) * d + e) * s - m[e];
          d2 += x * x;
        }
        if (d2 > best) best = d2;
      }
      r[(size_t)g * nb + J] = sqrt(best);
    }
  return 0;
}

/* qbar [hq][nb][d], kbar [hkv][nb][d], r [hkv][nb] -> rescue scores and
 * their row softmax, [hq][nb][nb], 0 above the diagonal (R may be NULL). */
int oracle_score_rescue(int hq, int hkv, int nb, int d, const double *qbar, const double *kbar,
                        const double *r, double c, double *R, double *Pr) {
  int grp = hq / hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int h = 0; h < hq; ++h)
    for (int I = 0; I < nb; ++I) {
      int g = h / grp;
      const double *qi = qbar + ((size_t)h * nb + I) * d;
      double *prow = Pr + ((size_t)h * nb + I) * nb;
      double qn = 0.0, m = -INFINITY, l = 0.0;
      for (int e = 0; e < d; ++e) qn += qi[e] * qi[e];
      qn = sqrt(qn);
      for (int J = 0; J < nb; ++J) prow[J] = 0.0;
      for (int J = 0; J <= I; ++J) {
        const double *kj = kbar + ((size_t)g * nb + J) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += qi[e] * kj[e];
        prow[J] = c * (dot + qn * r[(size_t)g * nb + J]);
        if (prow[J] > m) m = prow[J];
      }
      if (R) {
        double *rrow = R + ((size_t)h * nb + I) * nb;
        for (int J = 0; J < nb; ++J) rrow[J] = J <= I ? prow[J] : 0.0;
      }
      for (int J = 0; J <= I; ++J) l += exp(prow[J] - m);
      for (int J = 0; J <= I; ++J) prow[J] = exp(prow[J] - m) / l;
    }
  return 0;
}

/* Both branches thresholded independently, then combined with the forced
 * blocks and the causal condition; compaction as in oracle_mask. */
int oracle_mask_dual(int hq, int nb, const double *P, const double *Pr, double gamma,
                     double gamma_r, int sink_blocks, int local_blocks, uint8_t *mask,
                     int32_t *idx, int32_t *cnt) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < hq; ++h)
    for (int I = 0; I < nb; ++I) {
      size_t row = (size_t)h * nb + I;
      double pmax = -INFINITY, rmax = -INFINITY;
      for (int J = 0; J <= I; ++J) {
        if (P[row * nb + J] > pmax) pmax = P[row * nb + J];
        if (Pr[row * nb + J] > rmax) rmax = Pr[row * nb + J];
      }
      int n = 0;
      for (int J = 0; J < nb; ++J) {
        int keep = J <= I && (P[row * nb + J] >= gamma * pmax || Pr[row * nb + J] >= gamma_r * rmax ||
                              J < sink_blocks || I - J < local_blocks);
        mask[row * nb + J] = (uint8_t)keep;
        if (keep) idx[row * nb + n++] = J;
      }
      for (int J = n; J < nb; ++J) idx[row * nb + J] = -1;
      cnt[row] = n;
    }
  return 0;
}
