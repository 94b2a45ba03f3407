/*
 * m3_oracle.c -- plain, slow CPU oracle (test infrastructure only).
 *
 * Sources of each definition (the pages, by title and section):
 *  [metal]  TensorFold PR #987 "MiniMax Music 3 on Metal": the precision list
 *           (bf16 activations rounded where torch rounds, fp32 norms; int8
 *           weight-only with a scale per row for the body and lm_head and per
 *           group of 128 for the depth decoder), "What it adds" (decode GEMVs
 *           with a SwiGLU variant; Philox counters in the draw), the frame
 *           bookkeeping paragraph and "Kernel contract".
 *  [hf]     diffusers issue #14486 "MiniMax Music 3 modular pipeline", item 3
 *           (sliced lm_head is identical to the masked full one; Gumbel-argmax
 *           in place of softmax + multinomial) and item 4 (lockstep rows).
 *  [ds]     rkmt.cn "MiniMax-Music3 ... DiffSynth-Studio": model overview
 *           (Qwen3 body 4096 x 36, 32/8 heads; RVQ depth decoder 4 layers,
 *           16 heads, 8 codebooks) and stage 2 (vocab mask to the audio
 *           codes, per-codebook depth draws, frame embedding fed back as the
 *           sum of embed_tokens and the RVQ audio embeddings times 8^-1/2).
 *
 * Built with -ffp-contract=off and without fast-math: every fp32 operation
 * in the sampler is one IEEE operation in the order written.
 */
#include "m3_oracle.h"

#include <math.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int m3o_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* bf16: the upper 16 bits of an IEEE binary32; 8 significant bits.     */
/* Rounding is defined on the real value: pick the nearest bf16, ties   */
/* to the even significand; NaN -> 0x7FC0 (torch's canonical NaN).      */
/* ------------------------------------------------------------------ */
uint16_t m3o_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  if (isinf(v)) return v > 0 ? 0x7F80 : 0xFF80;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  double a = fabs(v);
  int e;
  frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
  double r;
  if (e - 1 < -126) {
    /* below the normal range: bf16 subnormals are multiples of 2^-133 */
    r = ldexp(nearbyint(ldexp(a, 133)), -133);
  } else {
    /* 8 significant bits: multiples of 2^(e-8) */
    r = ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);
  }
  /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds past it
     is infinity */
  if (r >= ldexp(1.0, 128)) return v > 0 ? 0x7F80 : 0xFF80;
  float f = (float)r;           /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t b = (uint16_t)(u >> 16);
  return v < 0 ? (uint16_t)(b | 0x8000) : b;
}

double m3o_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

void m3o_f64_to_bf16_n(const double* v, uint16_t* out, size_t n) {
  #pragma omp parallel for schedule(static)
  for (long i = 0; i < (long)n; ++i) out[i] = m3o_f64_to_bf16(v[i]);
}

void m3o_f32_to_bf16_n(const float* v, uint16_t* out, size_t n) {
  #pragma omp parallel for schedule(static)
  for (long i = 0; i < (long)n; ++i) out[i] = m3o_f64_to_bf16((double)v[i]);
}

/* ------------------------------------------------------------------ */
/* RMSNorm ([metal] precision list: fp32 norms, bf16 activations).      */
/* The oracle evaluates r in float64; one bf16 rounding of x*r*gamma.   */
/* ------------------------------------------------------------------ */
/* The norm's steps, in the precision the Metal port's precision list gives
   (fp32 norms, bf16 activations): r comes from a sum of squares taken in
   float64 (each square of a bf16 is exact in float64, and so is their sum
   over the ranges activations take, whatever the order) and is rounded once
   to fp32; each element is then fl32(fl32(x * r) * gamma), two fp32
   products, rounded once to bf16.  Every step is a single IEEE operation, so
   the bf16 rounding decision of each element is fixed by the steps alone. */
float m3o_norm_r(const uint16_t* x, int K, float eps) {
  double ss = 0.0;
  for (int k = 0; k < K; ++k) {
    double v = m3o_bf16_to_f64(x[k]);
    ss += v * v;
  }
  return (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

uint16_t m3o_norm_elem(uint16_t x, float r, float gamma) {
  const float xr = (float)m3o_bf16_to_f64(x) * r;    /* exact conversion, one fp32 product */
  const float a = xr * gamma;                          /* the second fp32 product */
  return m3o_f64_to_bf16((double)a);
}

void m3o_rmsnorm(const uint16_t* x, int B, int K, int ldx, const float* gamma,
                 float eps, uint16_t* a, int lda) {
  for (int b = 0; b < B; ++b) {
    const uint16_t* xr = x + (size_t)b * ldx;
    uint16_t* ar = a + (size_t)b * lda;
    if (!gamma) {
      for (int k = 0; k < K; ++k) ar[k] = xr[k];
      continue;
    }
    const float r = m3o_norm_r(xr, K, eps);
    for (int k = 0; k < K; ++k) ar[k] = m3o_norm_elem(xr[k], r, gamma[k]);
  }
}

/* ------------------------------------------------------------------ */
/* int8 weight-only quantisation ([metal] precision list).              */
/* scale = absmax / 127 as one fp32 division; q = nearest integer of    */
/* W / scale (ties to even), clamped to [-127, 127]; an all-zero row or */
/* group gets scale 0 and q 0.                                           */
/* ------------------------------------------------------------------ */
static void quant_span(const uint16_t* w, int n, int8_t* q, float* s) {
  double amax = 0.0;
  for (int k = 0; k < n; ++k) {
    double v = fabs(m3o_bf16_to_f64(w[k]));
    if (v > amax) amax = v;
  }
  float sc = (float)amax / 127.0f;   /* amax is exact in fp32 */
  *s = sc;
  for (int k = 0; k < n; ++k) {
    if (sc == 0.0f) { q[k] = 0; continue; }
    double t = nearbyint(m3o_bf16_to_f64(w[k]) / (double)sc);
    if (t > 127.0) t = 127.0;
    if (t < -127.0) t = -127.0;
    q[k] = (int8_t)t;
  }
}

void m3o_quant_i8row(const uint16_t* W, int N, int K, int8_t* q, float* s) {
  #pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    quant_span(W + (size_t)n * K, K, q + (size_t)n * K, s + n);
}

void m3o_quant_i8g128(const uint16_t* W, int N, int K, int8_t* q, float* s) {
  int G = K / 128;
  #pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int g = 0; g < G; ++g)
      quant_span(W + (size_t)n * K + g * 128, 128, q + (size_t)n * K + g * 128,
                 s + (size_t)n * G + g);
}

/* ------------------------------------------------------------------ */
/* fp8 weight-only (the next format after int8: [hf] and [mm] list fp8  */
/* weight-only only as a result measured on another stack; the format   */
/* is a reading made here): OCP FP8 E4M3 -- sign, 4 exponent bits with */
/* bias 7, 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9;   */
/* S.1111.111 is NaN; there is no infinity; the largest finite is 448.  */
/* One fp32 scale per row: s = absmax / 448 as one fp32 division, q =   */
/* the nearest E4M3 value of W / s (ties to the even mantissa),         */
/* saturated to +-448; an all-zero row gets s = 0 and q = 0.            */
/* ------------------------------------------------------------------ */
double m3o_fp8_decode(uint8_t c) {
  int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? (double)m * ldexp(1.0, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sgn ? -v : v;
}

uint8_t m3o_fp8_encode(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t sgn = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return sgn | 0x7E;                 /* saturate at the largest finite */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal,
       whose code is 8 as well */
    return sgn | (uint8_t)nearbyint(a * 512.0);
  }
  int x;
  frexp(a, &x);                                      /* a = f 2^x, f in [0.5, 1) */
  int E = x - 1;                                     /* a in [2^E, 2^(E+1)) */
  double m = nearbyint((ldexp(a, -E) - 1.0) * 8.0);  /* exact scaling, then RNE */
  if (m == 8.0) { m = 0.0; E += 1; }
  int e = E + 7;
  if (e > 15 || (e == 15 && m == 7.0)) return sgn | 0x7E;
  return sgn | (uint8_t)(e << 3) | (uint8_t)m;
}

void m3o_quant_fp8row(const uint16_t* W, int N, int K, uint8_t* q, float* s) {
  #pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    const uint16_t* w = W + (size_t)n * K;
    double amax = 0.0;
    for (int k = 0; k < K; ++k) {
      double v = fabs(m3o_bf16_to_f64(w[k]));
      if (v > amax) amax = v;
    }
    float sc = (float)amax / 448.0f;   /* amax is exact in fp32 */
    s[n] = sc;
    for (int k = 0; k < K; ++k)
      q[(size_t)n * K + k] = sc == 0.0f ? 0 : m3o_fp8_encode(m3o_bf16_to_f64(w[k]) / (double)sc);
  }
}

/* ------------------------------------------------------------------ */
/* y = Wdeq . a, summed in float64.  Each bf16*bf16 product is exact in */
/* float64, int8*bf16 too; only the running sum rounds (at 2^-53).      */
/* ------------------------------------------------------------------ */
static double dot_row(const m3o_mat* m, int n, const uint16_t* a) {
  int K = m->K;
  if (m->fmt == M3O_BF16) {
    const uint16_t* w = m->w + (size_t)n * K;
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += m3o_bf16_to_f64(w[k]) * m3o_bf16_to_f64(a[k]);
    return acc;
  }
  if (m->fmt == M3O_FP8ROW) {
    const uint8_t* c = (const uint8_t*)m->q + (size_t)n * K;
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += m3o_fp8_decode(c[k]) * m3o_bf16_to_f64(a[k]);
    return (double)m->s[n] * acc;
  }
  const int8_t* q = m->q + (size_t)n * K;
  if (m->fmt == M3O_I8ROW) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += (double)q[k] * m3o_bf16_to_f64(a[k]);
    return (double)m->s[n] * acc;
  }
  int G = K / 128;
  double acc = 0.0;
  for (int g = 0; g < G; ++g) {
    double part = 0.0;
    for (int k = g * 128; k < g * 128 + 128; ++k)
      part += (double)q[k] * m3o_bf16_to_f64(a[k]);
    acc += (double)m->s[(size_t)n * G + g] * part;
  }
  return acc;
}

void m3o_gemv_rows(const m3o_mat* m, int row0, int nrows, const uint16_t* a,
                   int B, int lda, double* y) {
  #pragma omp parallel for schedule(static)
  for (int n = 0; n < nrows; ++n)
    for (int b = 0; b < B; ++b)
      y[(size_t)b * nrows + n] = dot_row(m, row0 + n, a + (size_t)b * lda);
}

void m3o_gemv(const m3o_mat* m, const uint16_t* a, int B, int lda, double* y) {
  m3o_gemv_rows(m, 0, m->N, a, B, lda, y);
}

/* ------------------------------------------------------------------ */
/* Epilogues.  SwiGLU from an interleaved gate/up pair ([metal] "What   */
/* it adds": a gate and an up row whose SwiGLU is written together).    */
/* g and u are the bf16-rounded products; silu(g)*u is rounded once.    */
/* ------------------------------------------------------------------ */
void m3o_swiglu_interleaved(const double* y, int B, int F, uint16_t* m) {
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < F; ++i) {
      double g = m3o_bf16_to_f64(m3o_f64_to_bf16(y[(size_t)b * 2 * F + 2 * i]));
      double u = m3o_bf16_to_f64(m3o_f64_to_bf16(y[(size_t)b * 2 * F + 2 * i + 1]));
      m[(size_t)b * F + i] = m3o_f64_to_bf16(g * u / (1.0 + exp(-g)));
    }
}

void m3o_residual(const double* y, const uint16_t* h, int n, uint16_t* h_out) {
  for (int i = 0; i < n; ++i) {
    double yb = m3o_bf16_to_f64(m3o_f64_to_bf16(y[i]));
    h_out[i] = m3o_f64_to_bf16(m3o_bf16_to_f64(h[i]) + yb);
  }
}

/* Identity attention: with one cached position the softmax over one key is
   exactly 1, so each query head's output is its KV group's value head. */
void m3o_attn_stub(const uint16_t* qkv, int B, int ldq, int voff, int n_heads,
                   int group, int hd, uint16_t* o) {
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < n_heads; ++h)
      for (int d = 0; d < hd; ++d)
        o[(size_t)b * n_heads * hd + h * hd + d] =
            qkv[(size_t)b * ldq + voff + (h / group) * hd + d];
}

/* ------------------------------------------------------------------ */
/* Decode attention ("MiniMax Music 3, local" and TensorFold PR #987's    */
/* kernel list: per-head q/k norm and RoPE, decode attention over the     */
/* cached keys, the depth decoder's attention over its codebook positions;*/
/* the precision contract there: fp32 norms, softmax, rope and attention  */
/* sums with bf16 activations).  The body is Qwen3-shaped: RoPE base 1e6, */
/* rotation of the pairs (i, i + hd/2).                                   */
/* ------------------------------------------------------------------ */
void m3o_rope_table(int max_pos, int head_dim, double theta, float* t) {
  const int half = head_dim / 2;
  for (int p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = pow(theta, -(double)i / (double)half);
      const double ang = (double)p * inv;
      t[((size_t)p * half + i) * 2] = (float)cos(ang);
      t[((size_t)p * half + i) * 2 + 1] = (float)sin(ang);
    }
}

/* RMSNorm of one head's hd values, then its rotation at position pos */
static void norm_rope_head(const uint16_t* x, int hd, const float* gamma, float eps,
                           const float* rope_pos, uint16_t* y) {
  const int half = hd / 2;
  uint16_t xn[512];
  /* the head's RMSNorm: the same steps as m3o_rmsnorm */
  const float r = m3o_norm_r(x, hd, eps);
  for (int d = 0; d < hd; ++d) xn[d] = m3o_norm_elem(x[d], r, gamma[d]);
  for (int i = 0; i < half; ++i) {
    const double c = (double)rope_pos[2 * i], s = (double)rope_pos[2 * i + 1];
    const double a = m3o_bf16_to_f64(xn[i]), b = m3o_bf16_to_f64(xn[i + half]);
    y[i] = m3o_f64_to_bf16(a * c - b * s);
    y[i + half] = m3o_f64_to_bf16(b * c + a * s);
  }
}

void m3o_qk_norm_rope(const uint16_t* qkv, int B, int ldq, int n_q, int n_kv, int hd,
                      const float* q_gamma, const float* k_gamma, float eps, const float* rope,
                      int pos, uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                      int max_pos) {
  const float* rp = rope + (size_t)pos * (hd / 2) * 2;
  for (int b = 0; b < B; ++b) {
    const uint16_t* row = qkv + (size_t)b * ldq;
    for (int h = 0; h < n_q; ++h)
      norm_rope_head(row + h * hd, hd, q_gamma, eps, rp, q_out + ((size_t)b * n_q + h) * hd);
    for (int h = 0; h < n_kv; ++h) {
      const size_t slot = (((size_t)b * n_kv + h) * max_pos + pos) * hd;
      norm_rope_head(row + (n_q + h) * hd, hd, k_gamma, eps, rp, k_cache + slot);
      for (int d = 0; d < hd; ++d) v_cache[slot + d] = row[(n_q + n_kv + h) * hd + d];
    }
  }
}

void m3o_decode_attention(const uint16_t* q, int B, int n_q, int n_kv, int hd,
                          const uint16_t* k_cache, const uint16_t* v_cache, int max_pos, int T,
                          uint16_t* out) {
  const int g = n_q / n_kv;
  const double scale = 1.0 / sqrt((double)hd);
  double* sc = (double*)malloc(sizeof(double) * (size_t)T);
  double acc[512];
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < n_q; ++h) {
      const uint16_t* qh = q + ((size_t)b * n_q + h) * hd;
      const size_t base = ((size_t)b * n_kv + h / g) * max_pos * hd;
      double mx = -INFINITY;
      for (int t = 0; t < T; ++t) {
        const uint16_t* kt = k_cache + base + (size_t)t * hd;
        double dot = 0.0;
        for (int d = 0; d < hd; ++d) dot += m3o_bf16_to_f64(qh[d]) * m3o_bf16_to_f64(kt[d]);
        sc[t] = dot * scale;
        if (sc[t] > mx) mx = sc[t];
      }
      double sum = 0.0;
      for (int t = 0; t < T; ++t) {
        sc[t] = exp(sc[t] - mx);
        sum += sc[t];
      }
      for (int d = 0; d < hd; ++d) acc[d] = 0.0;
      for (int t = 0; t < T; ++t) {
        const uint16_t* vt = v_cache + base + (size_t)t * hd;
        for (int d = 0; d < hd; ++d) acc[d] += sc[t] * m3o_bf16_to_f64(vt[d]);
      }
      for (int d = 0; d < hd; ++d) out[((size_t)b * n_q + h) * hd + d] = m3o_f64_to_bf16(acc[d] / sum);
    }
  free(sc);
}

/* ------------------------------------------------------------------ */
/* Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:*/
/* As Easy as 1, 2, 3", SC'11): 10 rounds of two 32x32->64 multiplies   */
/* (multipliers 0xD2511F53, 0xCD9E8D57) with a Weyl key schedule        */
/* (0x9E3779B9, 0xBB67AE85).                                             */
/* ------------------------------------------------------------------ */
void m3o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Natural log of a positive normal fp32, from the identity
   ln x = e ln2 + 2 atanh(t), x = m 2^e, m in (1/sqrt2, sqrt2], t = (m-1)/(m+1),
   2 atanh t = 2 (t + t^3/3 + t^5/5 + t^7/7 + t^9/9 + t^11/11 + ...).
   |t| <= 0.1716, so the first omitted term is below 2^-36 relative.
   Every step is one IEEE fp32 operation (fmaf is the fused one). */
float m3o_logf(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  int e = (int)((u >> 23) & 0xFFu) - 127;
  uint32_t mb = (u & 0x007FFFFFu) | 0x3F800000u;
  float m;
  memcpy(&m, &mb, 4);                       /* m in [1, 2) */
  if (m > 1.41421354f) { m = m * 0.5f; e = e + 1; }
  float f = m - 1.0f;                       /* exact */
  float d = m + 1.0f;
  float t = f / d;
  float s = t * t;
  float p = 0.0909090936f;                  /* 1/11 */
  p = fmaf(p, s, 0.111111112f);             /* 1/9  */
  p = fmaf(p, s, 0.142857149f);             /* 1/7  */
  p = fmaf(p, s, 0.200000003f);             /* 1/5  */
  p = fmaf(p, s, 0.333333343f);             /* 1/3  */
  float sp = s * p;
  float r = sp * t;
  float lm = t + r;
  lm = lm + lm;
  float ef = (float)e;
  float res = fmaf(ef, 1.42860677e-06f, lm);   /* ln2 - ln2_hi */
  res = fmaf(ef, 0.693145752f, res);           /* ln2_hi = 0x3F317200 */
  return res;
}

/* Uniform on (0,1): the top 23 bits k of the word give the midpoint of the
   k-th of 2^23 equal cells, (k + 1/2) 2^-23 = (2k+1) 2^-24, exact in fp32. */
float m3o_uniform_from_word(uint32_t w) {
  uint32_t k = ((w >> 9) << 1) | 1u;       /* odd, < 2^24 */
  return (float)k * 5.96046448e-08f;        /* 2^-24 */
}

/* Gumbel noise keyed by (seed, batch row, frame, draw, absolute id). */
float m3o_gumbel(uint64_t seed, uint32_t row, uint32_t frame, uint32_t draw,
                 uint32_t id) {
  uint32_t ctr[4] = {id >> 2, row, frame, draw};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  m3o_philox4x32_10(ctr, key, w);
  float uu = m3o_uniform_from_word(w[id & 3u]);
  float l1 = m3o_logf(uu);        /* < 0 */
  float l2 = m3o_logf(-l1);
  return -l2;
}

/* total order used by the argmax: NaN above everything, then numeric;
   returns 1 if (za) ranks strictly above (zb) */
static int ranks_above(float za, float zb) {
  if (isnan(za)) return !isnan(zb);
  if (isnan(zb)) return 0;
  return za > zb;
}

/* Gumbel-argmax ([hf] item 3): argmax_j (l_j/T + G_j) draws j with
   probability softmax(l/T)_j.  Ties go to the lowest index. */
void m3o_gumbel_argmax(const float* logits, int B, int V, int ldl,
                       const m3o_sample_params* p, int32_t* out,
                       float* zbest, float* zsecond) {
  float invT = 1.0f / p->temperature;
  for (int b = 0; b < B; ++b) {
    int best = -1;
    float zb = 0.0f, z2 = -INFINITY;
    for (int j = 0; j < V; ++j) {
      int32_t id = p->ids ? p->ids[j] : p->index_base + j;
      float z;
      if (p->valid_lo < p->valid_hi && (id < p->valid_lo || id >= p->valid_hi)) {
        z = -INFINITY;
      } else {
        float g = p->noise_override ? p->noise_override[(size_t)b * V + j]
                                    : m3o_gumbel(p->seed, (uint32_t)b, p->frame,
                                                 p->draw, (uint32_t)id);
        float lt = logits[(size_t)b * ldl + j] * invT;
        z = lt + g;
      }
      if (best < 0 || ranks_above(z, zb)) {
        if (best >= 0) z2 = zb;
        best = j; zb = z;
      } else if (ranks_above(z, z2)) {
        z2 = z;
      }
    }
    out[b] = p->ids ? p->ids[best] : p->index_base + best;
    if (zbest) zbest[b] = zb;
    if (zsecond) zsecond[b] = z2;
  }
}

/* ------------------------------------------------------------------ */
/* The reference's own draw ([ds] stage 2: classifier-free guidance     */
/* with scale 1.5 over the conditional and unconditional rows, a top-k  */
/* filter with k = 50, then multinomial sampling; [metal] "What it      */
/* adds": the CFG top-k draw on the same Philox counters).              */
/*                                                                      */
/* Song s owns rows 2s (conditional, c) and 2s+1 (unconditional, u).    */
/*  1. guided g_j = u_j + fl32(scale * fl32(c_j - u_j)), three IEEE     */
/*     fp32 operations in this order; ids outside [valid_lo, valid_hi)  */
/*     and NaN guided values take no part;                              */
/*  2. the survivors are the k candidates with the largest g, ties      */
/*     to the lower column (all candidates when fewer than k);          */
/*  3. the multinomial draw from softmax(g/T) over the survivors is     */
/*     taken as Gumbel-argmax over them ([hf] item 3: the same law),    */
/*     z = fl32(g * fl32(1/T)) + G(seed, s, frame, draw, id), ranked    */
/*     as in the plain draw (NaN on top, ties to the lower column);     */
/*  4. the drawn id is written to both rows of the song.                */
/* A song without candidates draws its first column's id.               */
/* ------------------------------------------------------------------ */
typedef struct { float g; int j; } m3o_cand;

static int cand_order(const void* a, const void* b) {
  const m3o_cand* x = (const m3o_cand*)a;
  const m3o_cand* y = (const m3o_cand*)b;
  if (x->g > y->g) return -1;
  if (x->g < y->g) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

void m3o_cfg_topk_draw(const float* logits, int S, int V, int ldl, float scale, int top_k,
                       const m3o_sample_params* p, int32_t* out, int32_t* n_kept,
                       float* zgap) {
  float invT = 1.0f / p->temperature;
  m3o_cand* cand = (m3o_cand*)malloc((size_t)V * sizeof *cand);
  for (int s = 0; s < S; ++s) {
    const float* c = logits + (size_t)(2 * s) * ldl;
    const float* u = logits + (size_t)(2 * s + 1) * ldl;
    int n = 0;
    for (int j = 0; j < V; ++j) {
      int32_t id = p->ids ? p->ids[j] : p->index_base + j;
      if (p->valid_lo < p->valid_hi && (id < p->valid_lo || id >= p->valid_hi)) continue;
      float d = c[j] - u[j];
      float sd = scale * d;
      float g = u[j] + sd;
      if (isnan(g)) continue;
      cand[n].g = g;
      cand[n].j = j;
      ++n;
    }
    int keep = n < top_k ? n : top_k;
    int best = -1;
    float zb = 0.0f, z2 = -INFINITY;
    if (keep > 0) qsort(cand, (size_t)n, sizeof *cand, cand_order);
    for (int r = 0; r < keep; ++r) {
      int j = cand[r].j;
      int32_t id = p->ids ? p->ids[j] : p->index_base + j;
      float g = p->noise_override ? p->noise_override[(size_t)s * V + j]
                                  : m3o_gumbel(p->seed, (uint32_t)s, p->frame, p->draw,
                                               (uint32_t)id);
      float lt = cand[r].g * invT;
      float z = lt + g;
      /* the plain draw's order: NaN above every number, ties to the lower column */
      if (best < 0 || ranks_above(z, zb) || (!ranks_above(zb, z) && j < best)) {
        if (best >= 0) z2 = zb;
        best = j;
        zb = z;
      } else if (ranks_above(z, z2)) {
        z2 = z;
      }
    }
    if (best < 0) best = 0;
    int32_t id = p->ids ? p->ids[best] : p->index_base + best;
    out[2 * s] = id;
    out[2 * s + 1] = id;
    if (n_kept) n_kept[s] = keep;
    if (zgap) zgap[s] = keep > 0 ? zb - z2 : INFINITY;
  }
  free(cand);
}

/* ------------------------------------------------------------------ */
/* One frame ([ds] stage 2; [metal] frame bookkeeping).                 */
/* ------------------------------------------------------------------ */
/* one layer's attention over a KV cache: the new position pos is written,
   positions 0 .. pos are attended (NULL: the identity stub) */
typedef struct {
  const float* rope;
  uint16_t* kc;
  uint16_t* vc;
  int max_pos, pos;
  uint16_t* qbuf;                /* [B, n_heads * hd] */
} m3o_attn_at;

static void run_layer(const m3o_layer* L, uint16_t* h, int B, int Hd, int n_heads,
                      int n_kv, int hd, int F, float eps, uint16_t* a, uint16_t* qkvb,
                      uint16_t* o, uint16_t* mm, double* y, const m3o_attn_at* at) {
  int nq = n_heads * hd, nkv = n_kv * hd;
  int nqkv = nq + 2 * nkv;
  /* attention block */
  m3o_rmsnorm(h, B, Hd, Hd, L->attn_norm, eps, a, Hd);
  m3o_gemv(&L->qkv, a, B, Hd, y);
  m3o_f64_to_bf16_n(y, qkvb, (size_t)B * nqkv);
  if (at) {
    m3o_qk_norm_rope(qkvb, B, nqkv, n_heads, n_kv, hd, L->q_norm, L->k_norm, eps, at->rope,
                     at->pos, at->qbuf, at->kc, at->vc, at->max_pos);
    m3o_decode_attention(at->qbuf, B, n_heads, n_kv, hd, at->kc, at->vc, at->max_pos, at->pos + 1,
                         o);
  } else {
    m3o_attn_stub(qkvb, B, nqkv, nq + nkv, n_heads, n_heads / n_kv, hd, o);
  }
  m3o_gemv(&L->o, o, B, nq, y);
  m3o_residual(y, h, B * Hd, h);
  /* MLP block */
  m3o_rmsnorm(h, B, Hd, Hd, L->ffn_norm, eps, a, Hd);
  m3o_gemv(&L->gu, a, B, Hd, y);
  m3o_swiglu_interleaved(y, B, F, mm);
  m3o_gemv(&L->down, mm, B, F, y);
  m3o_residual(y, h, B * Hd, h);
}

/* The frame's draws: per row (Gumbel-argmax), or, with top_k > 0, the
   reference's draw over (conditional, unconditional) row pairs, one draw per
   song written to both of its rows ([ds] stage 2: guidance 1.5, top-k 50).
   zb - z2 receives each row's decision margin. */
static void draw_rows(const m3o_model* m, const float* lg, int B, int V,
                      const m3o_sample_params* p, int32_t* out, float* zb, float* z2) {
  if (m->top_k <= 0) {
    m3o_gumbel_argmax(lg, B, V, V, p, out, zb, z2);
    return;
  }
  int S = B / 2;
  float* gap = (float*)malloc((size_t)(S > 0 ? S : 1) * 4);
  m3o_cfg_topk_draw(lg, S, V, V, m->cfg_scale, m->top_k, p, out, NULL, gap);
  for (int b = 0; b < B; ++b) {
    zb[b] = gap[b / 2];
    z2[b] = 0.0f;
  }
  free(gap);
}

/* One layer with the identity attention stub, in place on h [B, Hd]: the
   step the frame takes per body layer and per depth layer ([ds] model
   overview; the benchmark workload stubs attention as identity). */
void m3o_layer_stub(const m3o_layer* L, uint16_t* h, int B, int Hd, int n_heads, int n_kv,
                    int hd, int F, float eps) {
  int nq = n_heads * hd, nkv = n_kv * hd;
  int wide = F > nq + 2 * nkv ? F : nq + 2 * nkv;
  double* y = (double*)malloc((size_t)B * (2 * (size_t)wide + 16) * sizeof(double));
  uint16_t* a = (uint16_t*)malloc((size_t)B * Hd * 2);
  uint16_t* qkvb = (uint16_t*)malloc((size_t)B * (nq + 2 * nkv) * 2);
  uint16_t* o = (uint16_t*)malloc((size_t)B * nq * 2);
  uint16_t* mm = (uint16_t*)malloc((size_t)B * F * 2);
  run_layer(L, h, B, Hd, n_heads, n_kv, hd, F, eps, a, qkvb, o, mm, y, NULL);
  free(y); free(a); free(qkvb); free(o); free(mm);
}

/* One layer with decode attention in place of the stub, in place on h: the
   layer's q/k norm + RoPE at position pos writes k and v to slot pos of the
   caches kc, vc ([B][n_kv][max_pos][hd]) and its heads attend over positions
   0 .. pos ("MiniMax Music 3, local" and TensorFold PR #987, kernel lists). */
void m3o_layer_attn(const m3o_layer* L, uint16_t* h, int B, int Hd, int n_heads, int n_kv, int hd,
                    int F, float eps, const float* rope, uint16_t* kc, uint16_t* vc, int max_pos,
                    int pos) {
  int nq = n_heads * hd, nkv = n_kv * hd;
  int wide = F > nq + 2 * nkv ? F : nq + 2 * nkv;
  double* y = (double*)malloc((size_t)B * (2 * (size_t)wide + 16) * sizeof(double));
  uint16_t* a = (uint16_t*)malloc((size_t)B * Hd * 2);
  uint16_t* qkvb = (uint16_t*)malloc((size_t)B * (nq + 2 * nkv) * 2);
  uint16_t* o = (uint16_t*)malloc((size_t)B * nq * 2);
  uint16_t* mm = (uint16_t*)malloc((size_t)B * F * 2);
  uint16_t* qbuf = (uint16_t*)malloc((size_t)B * nq * 2);
  m3o_attn_at at = {rope, kc, vc, max_pos, pos, qbuf};
  run_layer(L, h, B, Hd, n_heads, n_kv, hd, F, eps, a, qkvb, o, mm, y, &at);
  free(y); free(a); free(qkvb); free(o); free(mm); free(qbuf);
}

/* Input of depth step j ([ds] stage 2: the depth decoder draws codebook j
   from the frame's body state and the code drawn before it):
   hd[b] = bf16(u[b] + Emb_j[c_{j-1}]), with Emb_1 indexed by the semantic
   code's position in the slice (0 when outside it) and Emb_j, j >= 2, by the
   depth code of step j - 1.  codes: [B, 8] as the frame writes them. */
void m3o_step_input(const m3o_model* m, int j, const int32_t* codes, const uint16_t* u, int B,
                    uint16_t* hd) {
  int D = m->D;
  for (int b = 0; b < B; ++b) {
    int32_t prev;
    const uint16_t* E;
    if (j == 1) {
      prev = codes[b * 8] - m->vocab_base;
      if (prev < 0 || prev >= m->V0) prev = 0;
      E = m->emb1;
    } else {
      prev = codes[b * 8 + j - 1];
      E = m->emb[j - 2];
    }
    for (int k = 0; k < D; ++k)
      hd[(size_t)b * D + k] = m3o_f64_to_bf16(m3o_bf16_to_f64(u[(size_t)b * D + k]) +
                                              m3o_bf16_to_f64(E[(size_t)prev * D + k]));
  }
}

/* Next frame's input from the frame's 8 codes ([ds] stage 2: the codes are
   embedded, summed and scaled by the square root of the codebook count):
   x' = bf16((E_tok[c0] + sum_j A_j[c_j]) * 8^-1/2), summed in float64. */
void m3o_feedback(const m3o_model* m, const int32_t* codes, int B, uint16_t* x_next) {
  int H = m->H;
  double scale = 1.0 / sqrt((double)m->n_codebooks);
  for (int b = 0; b < B; ++b) {
    int32_t c0 = codes[b * 8] - m->vocab_base;
    if (c0 < 0 || c0 >= m->V0) c0 = 0;
    for (int k = 0; k < H; ++k) {
      double acc = m3o_bf16_to_f64(m->tok_emb_audio[(size_t)c0 * H + k]);
      for (int j = 1; j < m->n_codebooks; ++j)
        acc += m3o_bf16_to_f64(m->audio_emb[j - 1][(size_t)codes[b * 8 + j] * H + k]);
      x_next[(size_t)b * H + k] = m3o_f64_to_bf16(acc * scale);
    }
  }
}

void m3o_decode_frame(const m3o_model* m, const uint16_t* x_in, int B,
                      uint64_t seed, uint32_t frame, float temperature,
                      int32_t* codes, uint16_t* x_next, m3o_frame_trace* tr) {
  int H = m->H, D = m->D;
  int nq = m->n_heads * m->head_dim, nkv = m->n_kv_heads * m->head_dim;
  int dq = m->d_heads * m->d_head_dim;
  size_t big = (size_t)B * (size_t)(2 * (m->F > m->Fd ? m->F : m->Fd) + nq + 2 * nkv + 3 * dq + m->V0 + 17);
  double* y = (double*)malloc(big * sizeof(double));
  uint16_t* h = (uint16_t*)malloc((size_t)B * H * 2);
  uint16_t* a = (uint16_t*)malloc((size_t)B * (H > D ? H : D) * 2);
  uint16_t* qkvb = (uint16_t*)malloc((size_t)B * (nq + 2 * nkv + 3 * dq) * 2);
  uint16_t* o = (uint16_t*)malloc((size_t)B * (nq > dq ? nq : dq) * 2);
  uint16_t* mm = (uint16_t*)malloc((size_t)B * (m->F > m->Fd ? m->F : m->Fd) * 2);
  uint16_t* u = (uint16_t*)malloc((size_t)B * D * 2);
  uint16_t* hd = (uint16_t*)malloc((size_t)B * D * 2);
  float* lg = (float*)malloc((size_t)B * (m->V0 + 1 > m->code_vocab ? m->V0 + 1 : m->code_vocab) * 4);
  int32_t* draw_out = (int32_t*)malloc((size_t)B * 4);
  float* zb = (float*)malloc((size_t)B * 4);
  float* z2 = (float*)malloc((size_t)B * 4);

  uint16_t* qbuf = (uint16_t*)malloc((size_t)B * (nq > dq ? nq : dq) * 2);
  /* the body position of this frame (held below max_pos, as the GPU does) */
  long bpos = (long)m->pos0 + (long)frame;
  if (m->attention && bpos >= m->max_pos) bpos = m->max_pos - 1;

  memcpy(h, x_in, (size_t)B * H * 2);
  for (int l = 0; l < m->n_layers; ++l) {
    m3o_attn_at at = {m->rope, m->attention ? m->kcache[l] : NULL,
                      m->attention ? m->vcache[l] : NULL, m->max_pos, (int)bpos, qbuf};
    run_layer(&m->layers[l], h, B, H, m->n_heads, m->n_kv_heads, m->head_dim, m->F,
              m->eps, a, qkvb, o, mm, y, m->attention ? &at : NULL);
  }
  if (tr && tr->h_body) memcpy(tr->h_body, h, (size_t)B * H * 2);

  /* final norm -> sliced lm_head -> draw 0 over the reachable ids: the
     audio codes, and the end token when the model has it (its own row, its
     noise keyed by its id, which is below every code's) */
  int e = m->end_id >= 0 ? 1 : 0, VL = m->V0 + e;
  m3o_rmsnorm(h, B, H, H, m->final_norm, m->eps, a, H);
  m3o_gemv(&m->lm_head, a, B, H, y);
  for (size_t i = 0; i < (size_t)B * VL; ++i) lg[i] = (float)y[i];
  if (tr && tr->logits0) memcpy(tr->logits0, lg, (size_t)B * VL * 4);
  int32_t* ids = (int32_t*)malloc((size_t)VL * 4);
  for (int n = 0; n < VL; ++n) ids[n] = (e && n == 0) ? m->end_id : m->vocab_base + n - e;
  m3o_sample_params sp = {seed, frame, 0u, temperature, 0, ids, 0, 0, NULL};
  draw_rows(m, lg, B, VL, &sp, draw_out, zb, z2);
  free(ids);
  for (int b = 0; b < B; ++b) {
    codes[b * 8 + 0] = draw_out[b];
    if (tr && tr->zgap) tr->zgap[b * 8 + 0] = zb[b] - z2[b];
  }

  /* depth decoder input: u = bf16(P_in . normed body state) */
  m3o_gemv(&m->p_in, a, B, H, y);
  m3o_f64_to_bf16_n(y, u, (size_t)B * D);

  for (int j = 1; j < m->n_codebooks; ++j) {
    m3o_step_input(m, j, codes, u, B, hd);
    for (int l = 0; l < m->d_layers; ++l) {
      /* step j attends over the frame's codebook positions 0 .. j - 1 */
      m3o_attn_at at = {m->rope, m->attention ? m->dkcache[l] : NULL,
                        m->attention ? m->dvcache[l] : NULL, 8, j - 1, qbuf};
      run_layer(&m->d_layers_w[l], hd, B, D, m->d_heads, m->d_heads, m->d_head_dim, m->Fd,
                m->eps, a, qkvb, o, mm, y, m->attention ? &at : NULL);
    }
    m3o_rmsnorm(hd, B, D, D, m->d_final_norm, m->eps, a, D);
    m3o_gemv(&m->heads[j - 1], a, B, D, y);
    for (size_t i = 0; i < (size_t)B * m->code_vocab; ++i) lg[i] = (float)y[i];
    m3o_sample_params dp = {seed, frame, (uint32_t)j, temperature, 0, NULL, 0, 0, NULL};
    draw_rows(m, lg, B, m->code_vocab, &dp, draw_out, zb, z2);
    for (int b = 0; b < B; ++b) {
      codes[b * 8 + j] = draw_out[b];
      if (tr && tr->zgap) tr->zgap[b * 8 + j] = zb[b] - z2[b];
    }
  }

  m3o_feedback(m, codes, B, x_next);
  free(y); free(h); free(a); free(qkvb); free(o); free(mm); free(u); free(hd);
  free(lg); free(draw_out); free(zb); free(z2); free(qbuf);
}
