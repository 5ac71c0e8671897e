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
 *  - int4 KV cache (the same move taken one step further: two codes per
 *    byte, one fp32 scale per (token, kv head)): element 2i of a row is the
 *    low nibble of byte i and element 2i+1 the high nibble, each a signed
 *    4-bit two's complement number; the pages give no packing, this is a
 *    reading.
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

/* Code of element c of one row of a quantised cache (bits = 8 or 4, see the
 * readings above). */
static double code_value(const uint8_t* row, int c, int bits) {
  if (bits == 8) return (double)(int8_t)row[c];
  int nib = (c % 2 == 0) ? (int)(row[c / 2] & 15u) : (int)(row[c / 2] >> 4);
  if (nib >= 8) nib -= 16;
  return (double)nib;
}

/* One output row by the three passes above.  s is caller scratch of Skv
 * doubles.  Plain inputs come as double rows kbase/vbase (kv_stride apart);
 * a quantised cache as code rows kq/vq of row_bytes bytes with per-row
 * scales ks/vs, each element being code * scale. */
static void attend_row(const double* qrow, int d, double scale,
                       int64_t jlo, int64_t jhi,
                       const double* kbase, const double* vbase, int64_t kv_stride,
                       const uint8_t* kq, const uint8_t* vq, const float* ks, const float* vs,
                       int bits, double* s, double* orow, double* lse_out) {
  const int64_t row_bytes = bits == 8 ? d : d / 2;
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
      const uint8_t* kr = kq + j * row_bytes;
      double sc = (double)ks[j];
      for (c = 0; c < d; c++) acc += qrow[c] * (code_value(kr, c, bits) * sc);
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
      const uint8_t* vr = vq + j * row_bytes;
      double sc = (double)vs[j];
      for (c = 0; c < d; c++) orow[c] += p * (code_value(vr, c, bits) * sc);
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
      attend_row(qrow, d, scale, jlo, jhi, kb, vb, kv_stride, NULL, NULL, NULL, NULL, 0,
                 s, o + r * (int64_t)d, lse + r);
    }
    free(s);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Prefill over packed sequences of different lengths ([FA-3MOVES] names
 * variable-length batches as a CANN feature without a layout; the packed
 * layout with cumulative offsets is a reading).  Sequence b owns query rows
 * cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1 and attends only
 * within itself, with the causal / window rules above applied to its own
 * lengths (Sq_b = cu_q[b+1] - cu_q[b], Skv_b likewise).  Layouts:
 *   q [total_q, Hq, d], k and v [total_k, Hkv, d];  cu_q, cu_k [B+1],
 *   non-decreasing from 0 to total_q / total_k.
 * rows: nrows pairs (h, i) with i a packed query row.  o: nrows x d, lse: nrows.
 */
int oracle_fwd_varlen_rows(const double* q, const double* k, const double* v,
                           const int* cu_q, const int* cu_k,
                           int B, int Hq, int Hkv, int total_q, int total_k, int d,
                           double scale, int causal, int window,
                           const int64_t* rows, int64_t nrows,
                           double* o, double* lse, int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || total_q < 0 || total_k < 0 || d < 1 || Hq % Hkv != 0) return ORACLE_BAD_ARGS;
  if (window < 0 || (window > 0 && !causal)) return ORACLE_BAD_ARGS;
  if (!q || !k || !v || !cu_q || !cu_k || !rows || !o || !lse || nrows < 0) return ORACLE_BAD_ARGS;
  if (cu_q[0] != 0 || cu_k[0] != 0 || cu_q[B] != total_q || cu_k[B] != total_k) return ORACLE_BAD_ARGS;
  for (int b = 0; b < B; b++) {
    if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return ORACLE_BAD_ARGS;
  }
  for (int64_t r = 0; r < nrows; r++) {
    int64_t h = rows[2 * r], i = rows[2 * r + 1];
    if (h < 0 || h >= Hq || i < 0 || i >= total_q) return ORACLE_BAD_ARGS;
  }
  int group = Hq / Hkv;
  int64_t max_skv = 1;
  for (int b = 0; b < B; b++) {
    if (cu_k[b + 1] - cu_k[b] > max_skv) max_skv = cu_k[b + 1] - cu_k[b];
  }
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)max_skv);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; r++) {
      if (!s) continue;
      int64_t h = rows[2 * r], i = rows[2 * r + 1];
      int b = 0; /* the sequence holding packed row i */
      while (cu_q[b + 1] <= i) b++;
      int sq = cu_q[b + 1] - cu_q[b], skv = cu_k[b + 1] - cu_k[b];
      int64_t hk = h / group;
      int64_t jlo, jhi;
      visible_range(i - cu_q[b], sq, skv, causal, window, &jlo, &jhi);
      const double* qrow = q + (i * Hq + h) * (int64_t)d;
      int64_t kv_stride = (int64_t)Hkv * d;
      const double* kb = k + ((int64_t)cu_k[b] * Hkv + hk) * (int64_t)d;
      const double* vb = v + ((int64_t)cu_k[b] * Hkv + hk) * (int64_t)d;
      attend_row(qrow, d, scale, jlo, jhi, kb, vb, kv_stride, NULL, NULL, NULL, NULL, 0,
                 s, o + r * (int64_t)d, lse + r);
    }
    free(s);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Decode over a quantised KV cache: one new query token per sequence, every
 * cached key visible.  Layouts:
 *   q [B, Hq, d];  kq, vq [B, Hkv, Skv, row_bytes] codes (row_bytes = d for
 *   int8, d/2 for int4);  ks, vs [B, Hkv, Skv] fp32.
 * rows: nrows pairs (b, h).  o: nrows x d, lse: nrows.
 */
static int decode_rows(const double* q, const uint8_t* kq, const float* ks,
                       const uint8_t* vq, const float* vs, const int* seqlens,
                       int B, int Hq, int Hkv, int Skv, int d, double scale,
                       const int64_t* rows, int64_t nrows,
                       double* o, double* lse, int nthreads, int bits) {
  if (bad_shape(B, Hq, Hkv, 1, Skv, d)) return ORACLE_BAD_ARGS;
  if (bits == 4 && d % 2 != 0) return ORACLE_BAD_ARGS;
  if (!q || !kq || !ks || !vq || !vs || !rows || !o || !lse || nrows < 0) return ORACLE_BAD_ARGS;
  for (int64_t r = 0; r < nrows; r++) {
    int64_t b = rows[2 * r], h = rows[2 * r + 1];
    if (b < 0 || b >= B || h < 0 || h >= Hq) return ORACLE_BAD_ARGS;
  }
  if (seqlens) {
    for (int b = 0; b < B; b++) {
      if (seqlens[b] < 0 || seqlens[b] > Skv) return ORACLE_BAD_ARGS;
    }
  }
  int group = Hq / Hkv;
  int64_t row_bytes = bits == 8 ? d : d / 2;
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
      int64_t len = seqlens ? seqlens[b] : Skv; /* sequence b sees its first len cached tokens */
      attend_row(qrow, d, scale, 0, len, NULL, NULL, 0,
                 kq + stream * Skv * row_bytes, vq + stream * Skv * row_bytes,
                 ks + stream * Skv, vs + stream * Skv, bits,
                 s, o + r * (int64_t)d, lse + r);
    }
    free(s);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* int8 cache: kq, vq [B, Hkv, Skv, d] int8.  seqlens: NULL (every sequence
 * sees all Skv cached tokens) or [B] lengths, 0 <= seqlens[b] <= Skv (a
 * variable-length batch, [FA-3MOVES] CANN feature list). */
int oracle_decode_int8_rows(const double* q, const int8_t* kq, const float* ks,
                            const int8_t* vq, const float* vs, const int* seqlens,
                            int B, int Hq, int Hkv, int Skv, int d, double scale,
                            const int64_t* rows, int64_t nrows,
                            double* o, double* lse, int nthreads) {
  return decode_rows(q, (const uint8_t*)kq, ks, (const uint8_t*)vq, vs, seqlens, B, Hq, Hkv, Skv,
                     d, scale, rows, nrows, o, lse, nthreads, 8);
}

/* int4 cache: kq, vq [B, Hkv, Skv, d/2] bytes, two codes each; d even. */
int oracle_decode_int4_rows(const double* q, const uint8_t* kq, const float* ks,
                            const uint8_t* vq, const float* vs, const int* seqlens,
                            int B, int Hq, int Hkv, int Skv, int d, double scale,
                            const int64_t* rows, int64_t nrows,
                            double* o, double* lse, int nthreads) {
  return decode_rows(q, kq, ks, vq, vs, seqlens, B, Hq, Hkv, Skv, d, scale, rows, nrows, o, lse,
                     nthreads, 4);
}

/*
 * Appending tokens to a quantised KV cache: for every (b, t, kv head) row x
 * of d values, scale = absmax(x) / qmax and code_c = clamp(round(x_c /
 * scale), -qmax, qmax), round-half-to-even; an all-zero row gets scale 0
 * and codes 0.  qmax is 127 for the int8 cache and 7 for the int4 cache.
 * This is the per-(token, kv head) symmetric scheme of the quantised
 * workloads; [FA-3MOVES] move 3 names the int8 cache but gives no scheme.
 * Because the result is integer, the arithmetic deciding it is the kernel's:
 * IEEE fp32, one correctly rounded division for the scale and one per
 * element.
 *   x [B, T, Hkv, d] (float values; bf16 inputs are widened exactly)
 *   codes [B, Hkv, cap, row_bytes] (int8: d bytes; int4: d/2 bytes packed
 *   as in the readings above), scales [B, Hkv, cap] fp32: positions
 *   pos .. pos+T-1 are written, everything else is left as it was.
 */
static int kv_quantize(const float* x, uint8_t* codes, float* scales,
                       int B, int Hkv, int T, int d, int pos, int cap, float qmax, int bits) {
  if (B < 1 || Hkv < 1 || T < 1 || d < 1 || pos < 0 || (int64_t)pos + T > cap) return ORACLE_BAD_ARGS;
  if (bits == 4 && d % 2 != 0) return ORACLE_BAD_ARGS;
  if (!x || !codes || !scales) return ORACLE_BAD_ARGS;
  int64_t row_bytes = bits == 8 ? d : d / 2;
  for (int64_t b = 0; b < B; b++) {
    for (int64_t t = 0; t < T; t++) {
      for (int64_t h = 0; h < Hkv; h++) {
        const float* row = x + ((b * T + t) * Hkv + h) * (int64_t)d;
        float amax = 0.0f;
        for (int c = 0; c < d; c++) {
          float a = fabsf(row[c]);
          if (a > amax) amax = a;
        }
        volatile float scale = amax / qmax; /* stored as fp32, as the cache holds it */
        int64_t slot = (b * Hkv + h) * (int64_t)cap + pos + t;
        scales[slot] = scale;
        uint8_t* out = codes + slot * row_bytes;
        if (bits == 4) {
          for (int64_t i = 0; i < row_bytes; i++) out[i] = 0;
        }
        for (int c = 0; c < d; c++) {
          int code = 0;
          if (scale != 0.0f) {
            volatile float qv = row[c] / scale;
            float r = rintf(qv); /* default rounding mode: to nearest, ties to even */
            if (r > qmax) r = qmax;
            if (r < -qmax) r = -qmax;
            code = (int)r;
          }
          if (bits == 8) {
            out[c] = (uint8_t)(int8_t)code;
          } else {
            unsigned nib = (unsigned)code & 15u;
            out[c / 2] |= (uint8_t)(c % 2 == 0 ? nib : nib << 4);
          }
        }
      }
    }
  }
  return ORACLE_OK;
}

/* int8 cache: codes [B, Hkv, cap, d] int8, qmax 127. */
int oracle_kv_quantize_int8(const float* x, int8_t* codes, float* scales,
                            int B, int Hkv, int T, int d, int pos, int cap) {
  return kv_quantize(x, (uint8_t*)codes, scales, B, Hkv, T, d, pos, cap, 127.0f, 8);
}

/* int4 cache: codes [B, Hkv, cap, d/2] bytes, qmax 7; d even. */
int oracle_kv_quantize_int4(const float* x, uint8_t* codes, float* scales,
                            int B, int Hkv, int T, int d, int pos, int cap) {
  return kv_quantize(x, codes, scales, B, Hkv, T, d, pos, cap, 7.0f, 4);
}

/*
 * Backward pass: gradients of the forward above with respect to q, k and v,
 * for an upstream gradient dO of the output ([FA-NPU] recomputation section:
 * the backward pass recomputes the attention weights instead of storing
 * them).  Written out from the definition of the forward, with P_ij the
 * normalised probability of visible key j for query row i of head h:
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . V_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j  = scale * sum_i dS_ij Q_i
 * Masked keys have P_ij = 0 and receive nothing; a row with no visible key
 * contributes nothing and gets dQ_i = 0.  dK and dV of a kv head sum over the
 * query heads sharing it.  Layouts as oracle_fwd_rows; dO, dq like q; dk, dv
 * like k (all double).
 * o (may be NULL; laid out like q): a stored forward output.  When given,
 * D_i is formed from it as dO_i . O_i, the same quantity by the identity
 * sum_j P_ij (dO_i . V_j) = dO_i . (sum_j P_ij V_j) = dO_i . O_i; a backward
 * that starts from the saved output ([FA-NPU] recomputation section) sees
 * that output as it was stored, rounding included.
 * Pass 1 (one thread per query row): the row's P by the forward's three
 * passes, its dP, D_i and dQ_i; it keeps lse_i = m + log(l) and D_i.
 * Pass 2 (one thread per key of a kv head): P_ij = exp(scale q_i.k_j - lse_i),
 * the same weights, summed over the group's query rows in order (head, row).
 * Neither pass depends on the thread count.
 */
int oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
               const double* o, int B, int Hq, int Hkv, int Sq, int Skv, int d,
               double scale, int causal, int window,
               double* dq, double* dk, double* dv, int nthreads) {
  if (bad_shape(B, Hq, Hkv, Sq, Skv, d) || window < 0 || (window > 0 && !causal)) return ORACLE_BAD_ARGS;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return ORACLE_BAD_ARGS;
  int group = Hq / Hkv;
  int64_t nrows = (int64_t)B * Hq * Sq;
  int64_t kv_stride = (int64_t)Hkv * d;
  double* row_lse = (double*)malloc(sizeof(double) * (size_t)nrows);
  double* row_d = (double*)malloc(sizeof(double) * (size_t)nrows);
  if (!row_lse || !row_d) {
    free(row_lse);
    free(row_d);
    return ORACLE_NO_MEMORY;
  }
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  /* pass 1: rows (b, h, i) */
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)Skv);
    double* dp = (double*)malloc(sizeof(double) * (size_t)Skv);
    if (!p || !dp) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; r++) {
      if (!p || !dp) continue;
      int64_t b = r / ((int64_t)Hq * Sq), h = (r / Sq) % Hq, i = r % Sq;
      int64_t hk = h / group;
      const double* kh = k + (b * Skv * Hkv + hk) * (int64_t)d;
      const double* vh = v + (b * Skv * Hkv + hk) * (int64_t)d;
      const double* qi = q + ((b * Sq + i) * Hq + h) * (int64_t)d;
      const double* doi = dout + ((b * Sq + i) * Hq + h) * (int64_t)d;
      double* dqi = dq + ((b * Sq + i) * Hq + h) * (int64_t)d;
      int64_t jlo, jhi, j;
      int c;
      for (c = 0; c < d; c++) dqi[c] = 0.0;
      visible_range(i, Sq, Skv, causal, window, &jlo, &jhi);
      if (jhi <= jlo) {
        row_lse[r] = -INFINITY;
        row_d[r] = 0.0;
        continue;
      }
      double m = -INFINITY;
      for (j = jlo; j < jhi; j++) {
        double acc = 0.0;
        for (c = 0; c < d; c++) acc += qi[c] * kh[j * kv_stride + c];
        p[j - jlo] = scale * acc;
        if (p[j - jlo] > m) m = p[j - jlo];
      }
      double l = 0.0;
      for (j = jlo; j < jhi; j++) {
        p[j - jlo] = exp(p[j - jlo] - m);
        l += p[j - jlo];
      }
      for (j = jlo; j < jhi; j++) p[j - jlo] /= l;
      double D = 0.0;
      for (j = jlo; j < jhi; j++) {
        double acc = 0.0;
        for (c = 0; c < d; c++) acc += doi[c] * vh[j * kv_stride + c];
        dp[j - jlo] = acc;
        D += p[j - jlo] * acc;
      }
      if (o) {
        const double* oi = o + ((b * Sq + i) * Hq + h) * (int64_t)d;
        double Do = 0.0;
        for (c = 0; c < d; c++) Do += doi[c] * oi[c];
        D = Do;
      }
      for (j = jlo; j < jhi; j++) {
        double dsq = p[j - jlo] * (dp[j - jlo] - D);
        for (c = 0; c < d; c++) dqi[c] += scale * dsq * kh[j * kv_stride + c];
      }
      row_lse[r] = m + log(l);
      row_d[r] = D;
    }
    free(p);
    free(dp);
  }
  /* pass 2: keys (b, kv head, j), summing over the group's rows in order */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < (int64_t)B * Hkv * Skv; t++) {
    int64_t b = t / ((int64_t)Hkv * Skv), hk = (t / Skv) % Hkv, j = t % Skv;
    const double* kj = k + ((b * Skv + j) * Hkv + hk) * (int64_t)d;
    const double* vj = v + ((b * Skv + j) * Hkv + hk) * (int64_t)d;
    double* dkj = dk + ((b * Skv + j) * Hkv + hk) * (int64_t)d;
    double* dvj = dv + ((b * Skv + j) * Hkv + hk) * (int64_t)d;
    int c;
    for (c = 0; c < d; c++) {
      dkj[c] = 0.0;
      dvj[c] = 0.0;
    }
    for (int64_t h = hk * group; h < (hk + 1) * group; h++) {
      for (int64_t i = 0; i < Sq; i++) {
        int64_t jlo, jhi;
        visible_range(i, Sq, Skv, causal, window, &jlo, &jhi);
        if (j < jlo || j >= jhi) continue;
        int64_t r = (b * Hq + h) * Sq + i;
        const double* qi = q + ((b * Sq + i) * Hq + h) * (int64_t)d;
        const double* doi = dout + ((b * Sq + i) * Hq + h) * (int64_t)d;
        double s = 0.0, dpij = 0.0;
        for (c = 0; c < d; c++) {
          s += qi[c] * kj[c];
          dpij += doi[c] * vj[c];
        }
        double pij = exp(scale * s - row_lse[r]);
        double dsk = pij * (dpij - row_d[r]);
        for (c = 0; c < d; c++) {
          dvj[c] += pij * doi[c];
          dkj[c] += scale * dsk * qi[c];
        }
      }
    }
  }
  free(row_lse);
  free(row_d);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
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
