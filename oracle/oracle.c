/*
 * fp64 CPU oracle for tiled exact attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this file's library.  It shares no code, header or constant with
 * the HIP library; it is deliberately plain and slow.
 *
 * Sources (web pages; cited by title and section):
 *  [FA-NPU]   "When Transformer meets the Ascend NPU: the memory-slimming
 *             secret of the FlashAttention operator" (ai6s.net/6a0d479d...)
 *  [FA-3MOVES] the untitled ai6s.net article on FlashAttention's three moves
 *             and CANN 8.0 -> 8.5 (ai6s.net/6a0d6a93...)
 *  [FA-VARIANTS] "The FlashAttention variant family: GQA, MQA and sparse
 *             attention, how to choose" (ai6s.net/6a17bd37...)
 *
 * What it computes is the plain definition of scaled-dot-product attention,
 * softmax(Q K^T / sqrt(d_k)) V ([FA-NPU], section on why attention is so
 * memory-hungry), evaluated the way the standard four-step implementation
 * does it ([FA-3MOVES], section on the memory-move trap of standard
 * attention: scores, scaling, softmax, probabilities times V), one output
 * row at a time:
 *   pass 1  s_j = scale * sum_c q_c k_jc  for every visible key, and m = max s_j
 *   pass 2  e_j = exp(s_j - m),  l = sum e_j
 *   pass 3  o_c = sum_j (e_j / l) v_jc,   lse = m + log(l)
 * All arithmetic is double, summation in ascending index order, libm exp/log,
 * no fast-math, no intrinsics.  OpenMP splits rows over threads; one thread
 * owns a whole row, so results do not depend on the thread count.
 *
 * Readings of the pages used here:
 *  - head sharing: query head h reads key/value head floor(h / (Hq/Hkv)),
 *    the mapping that repeat_interleave(Hq/Hkv) along the head axis produces
 *    ([FA-VARIANTS], section on GQA on the NPU: KV expansion).
 *  - causal mask, bottom-right aligned: key j is visible to query i iff
 *    j <= i + (Skv - Sq) ([FA-NPU], section on how to use it, causal=True;
 *    the pages only show Sq == Skv, where this is the usual lower triangle).
 *  - sliding window of W keys including the query's own position: visible iff
 *    0 <= i + (Skv - Sq) - j < W ([FA-VARIANTS], local window attention
 *    section: each token attends to its nearest W tokens, N*W connections).
 *    A window needs the causal mask; window > 0 without causal is rejected
 *    (return -1), as every mask on that page is built on a lower triangle.
 *  - masked keys are excluded (additive -inf), never NaN (the page's mask
 *    code multiplies -inf by 0 at allowed positions; the intent is 0 / -inf).
 *  - a row with no visible key returns o = 0 and lse = -inf.
 *  - int8 KV cache ([FA-3MOVES], move 3, KV compression fused into the
 *    kernel): the cache stores int8 codes and one fp32 scale per (token,
 *    kv head); the value attention sees is code * scale, formed here in
 *    double on the fly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_NO_MEMORY (-2)

/* Validates the shape arguments shared by both entry points. */
static int bad_shape(int B, int Hq, int Hkv, int Sq, int Skv, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || d < 1) return 1;
  if (Hq % Hkv != 0) return 1;
  return 0;
}

/* One output row by the three passes above.  s is caller scratch of Skv
 * doubles.  kv_at(j) returns pointers to key/value row j; scale factors of a
 * quantised cache are passed through kscale/vscale (1.0 for plain inputs). */
static void attend_row(const double* qrow, int d, double scale,
                       int64_t jlo, int64_t jhi,
                       const double* kbase, const double* vbase, int64_t kv_stride,
                       const int8_t* kq, const int8_t* vq, const float* ks, const float* vs,
                       double* s, double* orow, double* lse_out) {
  int c;
  int64_t j;
  if (jhi <= jlo) {
    for (c = 0; c < d; c++) orow[c] = 0.0;
    *lse_out = -INFINITY;
    return;
  }
  /* pass 1: scores and their maximum */
  double m = -INFINITY;
  for (j = jlo; j < jhi; j++) {
    double acc = 0.0;
    if (kbase) {
      const double* kr = kbase + j * kv_stride;
      for (c = 0; c < d; c++) acc += qrow[c] * kr[c];
    } else {
      const int8_t* kr = kq + j * (int64_t)d;
      double sc = (double)ks[j];
      for (c = 0; c < d; c++) acc += qrow[c] * ((double)kr[c] * sc);
    }
    s[j - jlo] = scale * acc;
    if (s[j - jlo] > m) m = s[j - jlo];
  }
  /* pass 2: exponentials and their sum */
  double l = 0.0;
  for (j = jlo; j < jhi; j++) {
    s[j - jlo] = exp(s[j - jlo] - m);
    l += s[j - jlo];
  }
  /* pass 3: normalised probabilities times V */
  for (c = 0; c < d; c++) orow[c] = 0.0;
  for (j = jlo; j < jhi; j++) {
    double p = s[j - jlo] / l;
    if (vbase) {
      const double* vr = vbase + j * kv_stride;
      for (c = 0; c < d; c++) orow[c] += p * vr[c];
    } else {
      const int8_t* vr = vq + j * (int64_t)d;
      double sc = (double)vs[j];
      for (c = 0; c < d; c++) orow[c] += p * ((double)vr[c] * sc);
    }
  }
  *lse_out = m + log(l);
}

/* Visible key range [jlo, jhi) of query position i (see the readings above). */
static void visible_range(int64_t i, int Sq, int Skv, int causal, int window,
                          int64_t* jlo, int64_t* jhi) {
  int64_t off = (int64_t)Skv - (int64_t)Sq;
  int64_t lo = 0, hi = Skv;
  if (causal) {
    int64_t last = i + off; /* last visible key */
    hi = last + 1;
    if (hi > Skv) hi = Skv;
    if (hi < 0) hi = 0;
    if (window > 0) {
      lo = last - window + 1;
      if (lo < 0) lo = 0;
    }
  }
  if (lo > hi) lo = hi;
  *jlo = lo;
  *jhi = hi;
}

/*
 * Prefill / general forward.  Layouts (row-major, contiguous):
 *   q [B, Sq, Hq, d], k and v [B, Skv, Hkv, d]  (batch, sequence, heads, dim;
 *   the order [FA-NPU] gives for Q/K/V in its usage section).
 * rows: nrows triples (b, h, i) selecting the output rows to compute.
 * o: nrows x d, lse: nrows (natural log of the sum of exp of scaled scores).
 */
int oracle_fwd_rows(const double* q, const double* k, const double* v,
                    int B, int Hq, int Hkv, int Sq, int Skv, int d,
                    double scale, int causal, int window,
                    const int64_t* rows, int64_t nrows,
                    double* o, double* lse, int nthreads) {
  if (bad_shape(B, Hq, Hkv, Sq, Skv, d) || window < 0 || (window > 0 && !causal)) return ORACLE_BAD_ARGS;
  if (!q || !k || !v || !rows || !o || !lse || nrows < 0) return ORACLE_BAD_ARGS;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Sq) return ORACLE_BAD_ARGS;
  }
  int group = Hq / Hkv;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; r++) {
      if (!s) continue;
      int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      int64_t hk = h / group;
      int64_t jlo, jhi;
      visible_range(i, Sq, Skv, causal, window, &jlo, &jhi);
      const double* qrow = q + ((b * Sq + i) * Hq + h) * (int64_t)d;
      int64_t kv_stride = (int64_t)Hkv * d;
      const double* kb = k + (b * Skv * Hkv + hk) * (int64_t)d;
      const double* vb = v + (b * Skv * Hkv + hk) * (int64_t)d;
      attend_row(qrow, d, scale, jlo, jhi, kb, vb, kv_stride, NULL, NULL, NULL, NULL,
                 s, o + r * (int64_t)d, lse + r);
    }
    free(s);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Decode over an int8 KV cache: one new query token per sequence, every
 * cached key visible.  Layouts:
 *   q [B, Hq, d];  kq, vq [B, Hkv, Skv, d] int8;  ks, vs [B, Hkv, Skv] fp32.
 * rows: nrows pairs (b, h).  o: nrows x d, lse: nrows.
 */
int oracle_decode_int8_rows(const double* q, const int8_t* kq, const float* ks,
                            const int8_t* vq, const float* vs,
                            int B, int Hq, int Hkv, int Skv, int d, double scale,
                            const int64_t* rows, int64_t nrows,
                            double* o, double* lse, int nthreads) {
  if (bad_shape(B, Hq, Hkv, 1, Skv, d)) return ORACLE_BAD_ARGS;
  if (!q || !kq || !ks || !vq || !vs || !rows || !o || !lse || nrows < 0) return ORACLE_BAD_ARGS;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t b = rows[2 * r], h = rows[2 * r + 1];
    if (b < 0 || b >= B || h < 0 || h >= Hq) return ORACLE_BAD_ARGS;
  }
  int group = Hq / Hkv;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; r++) {
      if (!s) continue;
      int64_t b = rows[2 * r], h = rows[2 * r + 1];
      int64_t hk = h / group;
      int64_t stream = b * Hkv + hk;
      const double* qrow = q + (b * Hq + h) * (int64_t)d;
      attend_row(qrow, d, scale, 0, Skv, NULL, NULL, 0,
                 kq + stream * Skv * (int64_t)d, vq + stream * Skv * (int64_t)d,
                 ks + stream * Skv, vs + stream * Skv,
                 s, o + r * (int64_t)d, lse + r);
    }
    free(s);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Appending tokens to the int8 KV cache: for every (b, t, kv head) row x of
 * d values, scale = absmax(x) / 127 and code_c = clamp(round(x_c / scale),
 * -127, 127), round-half-to-even; an all-zero row gets scale 0 and codes 0.
 * This is the per-(token, kv head) symmetric scheme of the int8 workload;
 * [FA-3MOVES] move 3 names the int8 cache but gives no scheme.  Because the
 * result is integer, the arithmetic deciding it is the kernel's: IEEE fp32,
 * one correctly rounded division for the scale and one per element.
 *   x [B, T, Hkv, d] (float values; bf16 inputs are widened exactly)
 *   codes [B, Hkv, cap, d] int8, scales [B, Hkv, cap] fp32: positions
 *   pos .. pos+T-1 are written, everything else is left as it was.
 */
int oracle_kv_quantize_int8(const float* x, int8_t* codes, float* scales,
                            int B, int Hkv, int T, int d, int pos, int cap) {
  if (B < 1 || Hkv < 1 || T < 1 || d < 1 || pos < 0 || (int64_t)pos + T > cap) return ORACLE_BAD_ARGS;
  if (!x || !codes || !scales) return ORACLE_BAD_ARGS;
  for (int64_t b = 0; b < B; b++) {
    for (int64_t t = 0; t < T; t++) {
      for (int64_t h = 0; h < Hkv; h++) {
        const float* row = x + ((b * T + t) * Hkv + h) * (int64_t)d;
        float amax = 0.0f;
        for (int c = 0; c < d; c++) {
          float a = fabsf(row[c]);
          if (a > amax) amax = a;
        }
        volatile float scale = amax / 127.0f; /* stored as fp32, as the cache holds it */
        int64_t slot = (b * Hkv + h) * (int64_t)cap + pos + t;
        scales[slot] = scale;
        int8_t* out = codes + slot * (int64_t)d;
        for (int c = 0; c < d; c++) {
          if (scale == 0.0f) {
            out[c] = 0;
            continue;
          }
          volatile float qv = row[c] / scale;
          float r = rintf(qv); /* default rounding mode: to nearest, ties to even */
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          out[c] = (int8_t)r;
        }
      }
    }
  }
  return ORACLE_OK;
}

/* Number of threads an OpenMP region will use (for reporting). */
int oracle_max_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}
