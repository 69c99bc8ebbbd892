/*
 * attn_ref.c -- plain fp64 CPU oracle for scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes (the plain definition of attention that FlashAttention-2
 * reaches exactly up to rounding; "Attention Is All You Need", scaled
 * dot-product attention, as named on the Colfax author page, "Introduction to
 * Transformers" entry, and on the FlashAttention-2-on-Hopper abstract):
 *
 *   for every batch b, query head h and query row i, over the keys j that
 *   row may see (all Nk keys; with the causal option, j <= i + Nk - Nq):
 *     s_j   = scale * sum_c q[i][c] * k[j][c]           (fp64)
 *     m     = max_j s_j
 *     l     = sum_j exp(s_j - m)
 *     O[c]  = sum_j exp(s_j - m) * v[j][c] / l
 *     lse   = m + ln(l)           (natural-log logsumexp of the scaled logits)
 *   A row that may see no key gets O = 0 and lse = -inf.
 *
 * The base problem follows the "Kernel Specification" section of the
 * "Flash Attention 2 from scratch on Ampere" Part 1 page: forward only,
 * non-causal, no dropout, equal query/key/value lengths, 16-bit (bf16 or
 * fp16) inputs.  The options widen it along the rows that page excludes:
 * causal masking (aligned so the last query row sees every key), unequal
 * query and key lengths, and grouped key/value heads (query head h reads
 * key/value head h / (Hq / Hkv), as in the MQA/GQA setting of the Colfax
 * FlashAttention-3 inference post).  Inputs arrive as raw 16-bit patterns and
 * are decoded exactly to fp64; nothing here rounds to 16 bits or to fp32.
 *
 * Layout: q is [B][Hq][Nq][d], k and v are [B][Hkv][Nk][d], all contiguous;
 * O is [rows][d] fp64 and lse is [rows] fp64, where rows are either all
 * B*Hq*Nq rows in order or the caller's sorted list of flat row ids
 * (b*Hq + h)*Nq + i.
 *
 * INT8 key/value cache.  The Colfax author page lists the post
 * "FlashAttention-3 for Inference: INT8 Quantization and Query Head Packing
 * for MQA/GQA" by title only, with a teaser about in-kernel pre-processing of
 * tensors; the scheme below is this oracle's reading of that title, not a
 * quotation.  Keys and values arrive as int8 codes with fp32 per-channel
 * scales of their key/value head:
 *     k[j][c] = ks[c] * kq[j][c],   v[j][c] = vs[c] * vq[j][c].
 * Each query row is quantized to int8 after the key scales are folded into
 * it, every step in IEEE binary32 (the function quantize_q_row below):
 *     u[c]  = f32(q[c] * ks[c]),   amax = max_c |u[c]|,
 *     qq[c] = amax > 0 ? clamp(rint(f32(u[c] * f32(127 / amax))), -127, 127) : 0
 *             (rint rounds half to even),
 *     sq    = f32(amax / 127).
 * The logits are s_j = scale * sq * sum_c qq[c] * kq[j][c] (an exact integer
 * dot product), and the softmax, O and lse follow the definition above with
 * the dequantized v.
 *
 * FP8 key/value cache.  The same scheme with 8-bit floating-point codes in
 * place of the integers (the second reading of the same title: gfx950 also
 * multiplies FP8 matrices): every code is an OCP FP8 E4M3 value (1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9; 0x7F and 0xFF are NaN; the largest finite magnitude is
 * 448), and
 *     k[j][c] = ks[c] * e4m3(kq[j][c]),   v[j][c] = vs[c] * e4m3(vq[j][c]),
 *     qq[c] = amax > 0 ? e4m3_rne(f32(u[c] * f32(448 / amax))) : 0,
 *     sq    = f32(amax / 448),
 * where e4m3_rne rounds to the nearest E4M3 value, ties to the code with an
 * even last mantissa bit (the sign kept, magnitudes above 448 saturating to
 * 448; the query codes never exceed 448 by more than binary32 rounding).
 * The logits are s_j = scale * sq * sum_c qq[c] * e4m3(kq[j][c]), computed
 * here exactly in fp64.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1 };

/* bf16 is the upper half of an IEEE binary32 pattern: exact in fp64. */
static double decode_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
static double decode_fp16(uint16_t bits) {
  int sign = bits >> 15;
  int expo = (bits >> 10) & 0x1f;
  int man = bits & 0x3ff;
  double mag;
  if (expo == 0)
    mag = ldexp((double)man, -24); /* subnormal: man * 2^-14 * 2^-10 */
  else if (expo == 31)
    mag = man ? NAN : INFINITY;
  else
    mag = ldexp((double)(1024 + man), expo - 25); /* (1 + man/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

static double decode(uint16_t bits, int dtype) {
  return dtype == ORACLE_BF16 ? decode_bf16(bits) : decode_fp16(bits);
}

int oracle_decode(const uint16_t* bits, int64_t n, int dtype, double* out) {
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode(bits[i], dtype);
  return 0;
}

/* OCP FP8 E4M3 (see the header): the exact value of a code. */
static double decode_e4m3(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7)
    mag = NAN;
  else if (e == 0)
    mag = ldexp((double)m, -9);          /* subnormal: (m / 8) * 2^-6 */
  else
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m / 8) * 2^(e - 7) */
  return sign ? -mag : mag;
}

/* The E4M3 code nearest to x (x not NaN): a binary search over the 127
 * non-negative finite values, which increase with the code; a tie goes to
 * the even code; magnitudes beyond 448 give 448; the sign of x (also of a
 * zero) becomes the sign bit. */
static uint8_t round_e4m3(float x) {
  const double a = fabs((double)x);
  int lo = 0, hi = 126; /* decode_e4m3(lo) <= a < decode_e4m3(hi), or a at an end */
  uint8_t code;
  if (a >= decode_e4m3(126)) {
    code = 126;
  } else {
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (decode_e4m3((uint8_t)mid) <= a)
        lo = mid;
      else
        hi = mid;
    }
    const double dl = a - decode_e4m3((uint8_t)lo), dh = decode_e4m3((uint8_t)hi) - a;
    code = (uint8_t)(dl < dh ? lo : dh < dl ? hi : ((lo & 1) == 0 ? lo : hi));
  }
  return signbit(x) ? (uint8_t)(code | 0x80) : code;
}

int oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = decode_e4m3(codes[i]);
  return 0;
}

int oracle_e4m3_round(const float* x, int64_t n, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(x[i])) return -1;
    codes[i] = round_e4m3(x[i]);
  }
  return 0;
}

/* The FP8 scheme's query quantization for one row (see the header): every
 * operation in binary32 up to the rounding to E4M3.  Writes the codes to
 * code_out (when not NULL) and their values to qq; returns sq. */
static float quantize_q_row_fp8(const double* q, const float* ks, int64_t d, double* qq,
                                uint8_t* code_out) {
  float top = 0.0f; /* largest |q * ks| of the row */
  for (int64_t c = 0; c < d; ++c) {
    const float uk = (float)q[c] * ks[c];
    top = fmaxf(top, fabsf(uk));
  }
  if (!(top > 0.0f)) {
    for (int64_t c = 0; c < d; ++c) {
      qq[c] = 0.0;
      if (code_out) code_out[c] = 0;
    }
    return 0.0f;
  }
  const float to448 = 448.0f / top;
  for (int64_t c = 0; c < d; ++c) {
    const float uk = (float)q[c] * ks[c];
    const uint8_t code = round_e4m3(uk * to448);
    qq[c] = decode_e4m3(code);
    if (code_out) code_out[c] = code;
  }
  return top / 448.0f;
}

/* The INT8 scheme's query quantization for one row (see the header): every
 * operation in binary32, rounding half to even.  q holds the decoded 16-bit
 * values (exact in binary32), ks the key scales of the row's key/value head;
 * writes the codes to qq and returns sq. */
static float quantize_q_row(const double* q, const float* ks, int64_t d, double* qq) {
  float amax = 0.0f;
  for (int64_t c = 0; c < d; ++c) {
    const float u = (float)q[c] * ks[c];
    if (fabsf(u) > amax) amax = fabsf(u);
  }
  if (!(amax > 0.0f)) {
    for (int64_t c = 0; c < d; ++c) qq[c] = 0.0;
    return 0.0f;
  }
  const float inv = 127.0f / amax;
  for (int64_t c = 0; c < d; ++c) {
    const float u = (float)q[c] * ks[c];
    float code = rintf(u * inv);
    if (code > 127.0f) code = 127.0f;
    if (code < -127.0f) code = -127.0f;
    qq[c] = (double)code;
  }
  return amax / 127.0f;
}

/* Quantized codes and row scales of n query rows (16-bit patterns, d each),
 * all against the same key scales ks[d].  Returns 0, or -1 on a bad
 * argument. */
int oracle_quantize_q(const uint16_t* q, int dtype, int64_t n, int64_t d, const float* ks,
                      int8_t* qq, float* sq) {
  if ((dtype != ORACLE_BF16 && dtype != ORACLE_FP16) || n < 0 || d <= 0) return -1;
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  double* codes = (double*)malloc(sizeof(double) * (size_t)d);
  if (!row || !codes) {
    free(row);
    free(codes);
    return -1;
  }
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t c = 0; c < d; ++c) row[c] = decode(q[i * d + c], dtype);
    sq[i] = quantize_q_row(row, ks, d, codes);
    for (int64_t c = 0; c < d; ++c) qq[i * d + c] = (int8_t)codes[c];
  }
  free(row);
  free(codes);
  return 0;
}

/* The FP8 scheme's query codes and row scales, as oracle_quantize_q. */
int oracle_quantize_q_fp8(const uint16_t* q, int dtype, int64_t n, int64_t d, const float* ks,
                          uint8_t* qq, float* sq) {
  if ((dtype != ORACLE_BF16 && dtype != ORACLE_FP16) || n < 0 || d <= 0) return -1;
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  double* vals = (double*)malloc(sizeof(double) * (size_t)d);
  if (!row || !vals) {
    free(row);
    free(vals);
    return -1;
  }
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t c = 0; c < d; ++c) row[c] = decode(q[i * d + c], dtype);
    sq[i] = quantize_q_row_fp8(row, ks, d, vals, qq + i * d);
  }
  free(row);
  free(vals);
  return 0;
}

/* ------------------------------------------------------------------------ */

typedef struct {
  const uint16_t *q, *k, *v;
  const int8_t *kq, *vq;   /* INT8 cache codes (k, v unused then) */
  const uint8_t *kf, *vf;  /* FP8 (E4M3) cache codes (k, v unused then) */
  const float *ks, *vs;    /* their per-channel scales, [B][Hkv][d] */
  int dtype;
  int64_t B, Hq, Hkv, Nq, Nk, d;
  int causal;
  double scale;
  const int64_t* rows; /* sorted flat row ids, or NULL for all rows */
  int64_t nrows;
  double *o, *lse;
  int64_t chunk;           /* rows per work item */
  int64_t nitems;
  int64_t next;            /* shared work counter (guarded by mu) */
  int failed;              /* set by a worker that could not allocate */
  pthread_mutex_t mu;
} job_t;

/* One query row against the first N keys of one decoded head: the
 * definition, term by term.  N == 0 (no visible key) gives O = 0, lse = -inf. */
static void one_row(const double* qrow, const double* K, const double* V,
                    int64_t N, int64_t d, double scale, double* s,
                    double* orow, double* lse_out) {
  if (N <= 0) {
    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
    *lse_out = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < N; ++j) {
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qrow[c] * K[j * d + c];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    const double w = s[j];
    for (int64_t c = 0; c < d; ++c) orow[c] += w * V[j * d + c];
  }
  for (int64_t c = 0; c < d; ++c) orow[c] /= l;
  *lse_out = m + log(l);
}

/* Work item = (head, block of that head's selected rows). */
static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int64_t Nq = J->Nq, Nk = J->Nk, d = J->d;
  const int64_t group = J->Hq / J->Hkv;  /* query heads per key/value head */
  double* K = (double*)malloc(sizeof(double) * (size_t)(Nk * d + 1));
  double* V = (double*)malloc(sizeof(double) * (size_t)(Nk * d + 1));
  double* q = (double*)malloc(sizeof(double) * (size_t)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)(Nk + 1));
  int64_t loaded_head = -1;
  if (!K || !V || !q || !s) {
    pthread_mutex_lock(&J->mu);
    J->failed = 1;
    pthread_mutex_unlock(&J->mu);
    goto done;
  }
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t item = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (item >= J->nitems) break;
    int64_t r0 = item * J->chunk;
    int64_t r1 = r0 + J->chunk;
    if (r1 > J->nrows) r1 = J->nrows;
    for (int64_t r = r0; r < r1; ++r) {
      int64_t flat = J->rows ? J->rows[r] : r;
      int64_t head = flat / Nq, i = flat % Nq;  /* head = b*Hq + h */
      int64_t kv_head = (head / J->Hq) * J->Hkv + (head % J->Hq) / group;
      if (kv_head != loaded_head) {
        if (J->kf) {
          /* K holds the code values (the scales are folded into the query);
           * V the dequantized values, each an exact fp64 product */
          const uint8_t* kh = J->kf + kv_head * Nk * d;
          const uint8_t* vh = J->vf + kv_head * Nk * d;
          const float* vs = J->vs + kv_head * d;
          for (int64_t t = 0; t < Nk * d; ++t) {
            K[t] = decode_e4m3(kh[t]);
            V[t] = (double)vs[t % d] * decode_e4m3(vh[t]);
          }
        } else if (J->kq) {
          /* K holds the integer codes (the scales are folded into the
           * query); V the dequantized values, each an exact fp64 product */
          const int8_t* kh = J->kq + kv_head * Nk * d;
          const int8_t* vh = J->vq + kv_head * Nk * d;
          const float* vs = J->vs + kv_head * d;
          for (int64_t t = 0; t < Nk * d; ++t) {
            K[t] = (double)kh[t];
            V[t] = (double)vs[t % d] * (double)vh[t];
          }
        } else {
          const uint16_t* kh = J->k + kv_head * Nk * d;
          const uint16_t* vh = J->v + kv_head * Nk * d;
          for (int64_t t = 0; t < Nk * d; ++t) {
            K[t] = decode(kh[t], J->dtype);
            V[t] = decode(vh[t], J->dtype);
          }
        }
        loaded_head = kv_head;
      }
      /* keys 0 .. visible-1; causal rows are aligned so that the last query
       * row sees all Nk keys */
      int64_t visible = Nk;
      if (J->causal && i + 1 + Nk - Nq < visible) visible = i + 1 + Nk - Nq;
      const uint16_t* qr = J->q + flat * d;
      for (int64_t c = 0; c < d; ++c) q[c] = decode(qr[c], J->dtype);
      double row_scale = J->scale;
      if (J->kq) {  /* quantized query: codes in q, logits times sq */
        const float sq = quantize_q_row(q, J->ks + kv_head * d, d, q);
        row_scale = J->scale * (double)sq;
      } else if (J->kf) {  /* the same with E4M3 code values */
        const float sqf = quantize_q_row_fp8(q, J->ks + kv_head * d, d, q, NULL);
        row_scale = (double)sqf * J->scale;
      }
      one_row(q, K, V, visible, d, row_scale, s, J->o + r * d, J->lse + r);
    }
  }
done:
  free(K); free(V); free(q); free(s);
  return NULL;
}

int oracle_host_threads(void) {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  return 1;
}

/*
 * Attention rows, general form.  q [B][Hq][Nq][d], k and v [B][Hkv][Nk][d],
 * Hq a multiple of Hkv >= 1, causal 0 or 1.  rows == NULL computes all
 * B*Hq*Nq rows; otherwise rows[] is a strictly increasing list of nrows flat
 * row ids in [0, B*Hq*Nq).  nthreads <= 0 uses every core in the affinity
 * mask.  Returns 0, or -1 on a bad argument, -2 on allocation failure.
 */
static int run_job(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const int8_t* kq, const float* ks, const int8_t* vq, const float* vs,
                   const uint8_t* kf, const uint8_t* vf, int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                   int64_t d, double scale, int causal, const int64_t* rows, int64_t nrows,
                   double* o, double* lse, int nthreads) {
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return -1;
  if (B < 0 || Hq < 0 || Hkv <= 0 || Nq < 0 || Nk < 0 || d <= 0) return -1;
  if (Hq % Hkv != 0 || (causal != 0 && causal != 1)) return -1;
  const int64_t total = B * Hq * Nq;
  if (!rows) nrows = total;
  if (nrows < 0 || nrows > total) return -1;
  if (nrows == 0) return 0;
  if (!q || !o || !lse) return -1;
  if (kq || kf) {
    if (!ks || (Nk > 0 && (!(kq ? (const void*)vq : (const void*)vf) || !vs))) return -1;
  } else if (Nk > 0 && (!k || !v)) {
    return -1;
  }
  if (rows) {
    for (int64_t r = 0; r < nrows; ++r) {
      if (rows[r] < 0 || rows[r] >= total) return -1;
      if (r && rows[r] <= rows[r - 1]) return -1;
    }
  }
  if (nthreads <= 0) nthreads = oracle_host_threads();

  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.dtype = dtype;
  J.kq = kq; J.ks = ks; J.vq = vq; J.vs = vs;
  J.kf = kf; J.vf = vf;
  J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nk = Nk; J.d = d;
  J.causal = causal; J.scale = scale;
  J.rows = rows; J.nrows = nrows; J.o = o; J.lse = lse;
  /* rows of one head stay together inside an item so K/V decode once */
  J.chunk = 64;
  J.nitems = (nrows + J.chunk - 1) / J.chunk;
  if (J.nitems < nthreads && nrows >= nthreads) {
    J.chunk = (nrows + nthreads - 1) / nthreads;
    J.nitems = (nrows + J.chunk - 1) / J.chunk;
  }
  if (nthreads > J.nitems) nthreads = (int)J.nitems;
  pthread_mutex_init(&J.mu, NULL);

  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, &J) != 0) break;
    ++started;
  }
  if (started == 0) worker(&J);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return J.failed ? -2 : 0;
}

int oracle_attn_general(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                        int64_t Nk, int64_t d, double scale, int causal,
                        const int64_t* rows, int64_t nrows, double* o, double* lse,
                        int nthreads) {
  return run_job(q, k, v, NULL, NULL, NULL, NULL, NULL, NULL, dtype, B, Hq, Hkv, Nq, Nk, d,
                 scale, causal, rows, nrows, o, lse, nthreads);
}

/*
 * Attention over an INT8 key/value cache (the scheme in the header): q
 * [B][Hq][Nq][d] 16-bit patterns; kq, vq [B][Hkv][Nk][d] int8 codes; ks, vs
 * [B][Hkv][d] fp32 per-channel scales.  Rows, threads and the return codes
 * are those of oracle_attn_general.
 */
int oracle_attn_kv_int8(const uint16_t* q, int dtype, const int8_t* kq, const float* ks,
                        const int8_t* vq, const float* vs, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, double scale,
                        int causal, const int64_t* rows, int64_t nrows, double* o,
                        double* lse, int nthreads) {
  if (!kq) return -1;
  return run_job(q, NULL, NULL, kq, ks, vq, vs, NULL, NULL, dtype, B, Hq, Hkv, Nq, Nk, d, scale,
                 causal, rows, nrows, o, lse, nthreads);
}

/*
 * Attention over an FP8 (E4M3) key/value cache (the scheme in the header):
 * kf, vf [B][Hkv][Nk][d] E4M3 codes; everything else as oracle_attn_kv_int8.
 */
int oracle_attn_kv_fp8(const uint16_t* q, int dtype, const uint8_t* kf, const float* ks,
                       const uint8_t* vf, const float* vs, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, double scale,
                       int causal, const int64_t* rows, int64_t nrows, double* o,
                       double* lse, int nthreads) {
  if (!kf) return -1;
  return run_job(q, NULL, NULL, NULL, ks, NULL, vs, kf, vf, dtype, B, Hq, Hkv, Nq, Nk, d, scale,
                 causal, rows, nrows, o, lse, nthreads);
}

/* The base problem: equal heads and lengths, no mask. */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                     double scale, const int64_t* rows, int64_t nrows,
                     double* o, double* lse, int nthreads) {
  if (H <= 0) return (B >= 0 && H == 0 && N >= 0 && d > 0) ? 0 : -1;
  return oracle_attn_general(q, k, v, dtype, B, H, H, N, N, d, scale, 0, rows,
                             nrows, o, lse, nthreads);
}
