/*
 * m3_oracle.h -- CPU oracle for the per-frame autoregressive decode of a
 * MiniMax-Music-3-style audio LM (Qwen3-shaped body + RVQ depth decoder).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this code; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Every routine is plain scalar C in float64 unless a step is defined in fp32
 * by the method itself (the sampler).  Weights and activations are bf16 bit
 * patterns (uint16_t), fp32 scales/gammas are float.
 *
 * Parity pins: every function here is pinned by a CPU test that does not
 * re-use this code (exact rational brute force, closed forms, a library
 * routine, exhaustive sweeps).  The depth-decoder coupling inside
 * m3o_decode_frame is the one part whose interface the pages do not give:
 * "parity unpinned" for that coupling beyond its components.
 */
#ifndef M3_ORACLE_H
#define M3_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight formats (MiniMax Music 3 Metal port, precision section: bf16,
   int8 with one scale per row, int8 with one scale per group of 128) */
enum { M3O_BF16 = 0, M3O_I8ROW = 1, M3O_I8G128 = 2, M3O_FP8ROW = 3 };

/* ---- bf16 ---------------------------------------------------------- */
uint16_t m3o_f64_to_bf16(double v);      /* one round-to-nearest-even */
double   m3o_bf16_to_f64(uint16_t b);
void     m3o_f64_to_bf16_n(const double* v, uint16_t* out, size_t n);
void     m3o_f32_to_bf16_n(const float* v, uint16_t* out, size_t n);

/* ---- RMSNorm ------------------------------------------------------- */
/* a[b,k] = bf16( fl32(fl32(x[b,k] * r_b) * gamma[k]) ),
   r_b = fl32(1/sqrt(mean_k x^2 + eps)) with the sum and r in float64
   (fp32 norm arithmetic, the Metal port's precision list).
   gamma == NULL: a = x (no norm).  m3o_norm_r and m3o_norm_elem are its two
   steps (r of one row of K values; one element). */
void m3o_rmsnorm(const uint16_t* x, int B, int K, int ldx, const float* gamma,
                 float eps, uint16_t* a, int lda);
float m3o_norm_r(const uint16_t* x, int K, float eps);
uint16_t m3o_norm_elem(uint16_t x, float r, float gamma);

/* ---- int8 quantisers ------------------------------------------------ */
/* s_n = fl32(absmax_n / 127); q = clamp(rne(W/s), -127, 127); zero row: s=q=0 */
void m3o_quant_i8row(const uint16_t* W, int N, int K, int8_t* q, float* s);
/* the same per (row, group of 128 along K); s is [N, K/128] */
void m3o_quant_i8g128(const uint16_t* W, int N, int K, int8_t* q, float* s);

/* ---- fp8 weight-only (OCP FP8 E4M3, bias 7, no infinity, max 448) -- */
double  m3o_fp8_decode(uint8_t c);        /* NaN for S.1111.111 */
uint8_t m3o_fp8_encode(double v);         /* nearest, ties to even mantissa; |v| >= 448 -> +-448; NaN -> 0x7F */
/* s_n = fl32(absmax_n / 448); q = encode(W / s); zero row: s = q = 0 */
void m3o_quant_fp8row(const uint16_t* W, int N, int K, uint8_t* q, float* s);

/* ---- matrix-vector products (exact fp64 sums, unrounded) ------------ */
typedef struct {
  int fmt;              /* M3O_BF16 / M3O_I8ROW / M3O_I8G128 / M3O_FP8ROW */
  int N, K;
  const uint16_t* w;    /* bf16 [N,K]            (fmt == M3O_BF16) */
  const int8_t* q;      /* int8 [N,K] (int8 formats); fp8 codes [N,K] (M3O_FP8ROW) */
  const float* s;       /* [N] or [N, K/128]     (int8 and fp8 formats) */
} m3o_mat;

/* y[b*N + n] = sum_k Wdeq[n,k] * a[b,k]; Wdeq = w, s_n*q or s_{n,g}*q */
void m3o_gemv(const m3o_mat* m, const uint16_t* a, int B, int lda, double* y);
/* same, rows [row0, row0+nrows) only; y is [B, nrows] */
void m3o_gemv_rows(const m3o_mat* m, int row0, int nrows, const uint16_t* a,
                   int B, int lda, double* y);

/* ---- epilogues / attention stub ------------------------------------ */
/* g = bf16(y[b, 2i]) (gate), u = bf16(y[b, 2i+1]) (up) from interleaved rows;
   m[b, i] = bf16( g * u / (1 + exp(-g)) ) */
void m3o_swiglu_interleaved(const double* y, int B, int F, uint16_t* m);
/* h_out = bf16( h + bf16(y) ) */
void m3o_residual(const double* y, const uint16_t* h, int n, uint16_t* h_out);
/* identity attention: o[b, h*hd + d] = qkv[b, voff + (h/group)*hd + d] */
void m3o_attn_stub(const uint16_t* qkv, int B, int ldq, int voff, int n_heads,
                   int group, int hd, uint16_t* o);

/* ---- decode attention (q/k norm, RoPE, KV cache, softmax attention) --- */
/* RoPE table, theta^(-i/half) frequencies over pair i < half = head_dim/2:
 * t[(p*half + i)*2] = fl32(cos(p * theta^(-i/half))), [..+1] = fl32(sin(..)),
 * angle and trig in float64. */
void m3o_rope_table(int max_pos, int head_dim, double theta, float* t);
/* For every row b of qkv [B, ldq] (q heads at columns h*hd, k heads after the
 * n_q q heads, v heads after the k heads): per head RMSNorm over its hd values
 * (x' = bf16(x * r * gamma), as m3o_rmsnorm), then the rotation of pairs
 * (i, i + hd/2) by the table's angle of position pos:
 *   y_i = bf16(x'_i c - x'_{i+half} s),  y_{i+half} = bf16(x'_{i+half} c + x'_i s)
 * (float64 from the fp32 c, s).  q goes to q_out [B, n_q*hd]; k and the raw v
 * go to the caches [B][n_kv][max_pos][hd] at position pos. */
void m3o_qk_norm_rope(const uint16_t* qkv, int B, int ldq, int n_q, int n_kv, int hd,
                      const float* q_gamma, const float* k_gamma, float eps, const float* rope,
                      int pos, uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                      int max_pos);
/* out[b, h*hd + d] = bf16( sum_{t<T} p_t * v[b][h/g][t][d] ),
 * p = softmax_t( q[b,h] . k[b][h/g][t] / sqrt(hd) ), g = n_q / n_kv;
 * float64 throughout, one rounding. */
void m3o_decode_attention(const uint16_t* q, int B, int n_q, int n_kv, int hd,
                          const uint16_t* k_cache, const uint16_t* v_cache, int max_pos, int T,
                          uint16_t* out);

/* ---- sampler -------------------------------------------------------- */
void  m3o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
float m3o_logf(float x);                       /* fixed-sequence fp32 log   */
float m3o_uniform_from_word(uint32_t w);       /* (2*(w>>9)+1) * 2^-24      */
float m3o_gumbel(uint64_t seed, uint32_t row, uint32_t frame, uint32_t draw,
                 uint32_t id);
typedef struct {
  uint64_t seed; uint32_t frame; uint32_t draw; float temperature;
  int32_t index_base; const int32_t* ids; int32_t valid_lo, valid_hi;
  const float* noise_override;   /* [B, V] (row stride V) or NULL */
} m3o_sample_params;
/* out[b] = absolute id of argmax_j z[b,j]; z = fl32(l*fl32(1/T)) + g.
   zbest/zsecond (optional) receive the best and second-best z of each row
   (used by tests to measure how close a decision was). */
void m3o_gumbel_argmax(const float* logits, int B, int V, int ldl,
                       const m3o_sample_params* p, int32_t* out,
                       float* zbest, float* zsecond);
/* CFG + top-k draw over song pairs (rows 2s conditional, 2s+1
   unconditional): guided g = u + scale (c - u), the top_k largest g (ties to
   the lower column), Gumbel-argmax over them with counter row s; out[2s] =
   out[2s+1] = the drawn id.  n_kept (optional [S]) receives the survivor count,
   zgap (optional [S]) the best survivor's z minus the second best (inf with
   one survivor). */
void m3o_cfg_topk_draw(const float* logits, int S, int V, int ldl, float scale, int top_k,
                       const m3o_sample_params* p, int32_t* out, int32_t* n_kept,
                       float* zgap);

/* ---- one decode frame ------------------------------------------------ */
typedef struct {
  m3o_mat qkv, o, gu, down;      /* gu: interleaved gate/up rows [2F, H] */
  const float* attn_norm; const float* ffn_norm;
  const float* q_norm; const float* k_norm;   /* [head_dim]; attention only */
} m3o_layer;

typedef struct {
  /* body */
  int H, n_layers, n_heads, n_kv_heads, head_dim, F;
  const m3o_layer* layers;
  const float* final_norm;
  m3o_mat lm_head;               /* the reachable slice only [V0, H]  */
  int32_t vocab_base;            /* absolute id of slice row 0 (151675) */
  int V0;                        /* rows in the slice (16384)           */
  /* depth decoder */
  int D, d_layers, d_heads, d_head_dim, Fd, n_codebooks, code_vocab;
  m3o_mat p_in;                  /* [D, H] */
  const uint16_t* emb1;          /* [V0, D] semantic code embedding     */
  const uint16_t* const* emb;    /* emb[j-2], j = 2..7: [code_vocab, D] */
  const m3o_layer* d_layers_w;
  const float* d_final_norm;
  const m3o_mat* heads;          /* heads[j-1], [code_vocab, D]         */
  /* feedback */
  const uint16_t* tok_emb_audio; /* [V0, H]: embed_tokens rows of the audio codes */
  const uint16_t* const* audio_emb; /* audio_emb[j-1], [code_vocab, H]  */
  float eps;
  /* draws: top_k == 0 per row; top_k > 0 the reference's draw over row
     pairs (B even) with guidance scale cfg_scale ([ds] stage 2) */
  float cfg_scale;
  int top_k;
  /* attention: 0 the identity stub; 1 decode attention (m3o_qk_norm_rope,
     m3o_decode_attention) with frame f at body position pos0 + f over the
     caches kcache[l], vcache[l] ([B][n_kv][max_pos][hd], kept across frames),
     and the depth decoder's step j at position j - 1 over dkcache[l],
     dvcache[l] ([B][d_heads][8][d_head_dim], rewritten every frame); rope is
     an m3o_rope_table of at least max(max_pos, 8) positions */
  int attention, max_pos, pos0;
  const float* rope;
  uint16_t* const* kcache;
  uint16_t* const* vcache;
  uint16_t* const* dkcache;
  uint16_t* const* dvcache;
  /* the end token ([ds] stage 2: the semantic draw is masked to the audio
     codes and the end token, and a song ends when it is drawn): end_id < 0
     none; else lm_head has V0 + 1 rows, row 0 the end token's (id end_id)
     and row 1 + i code i's */
  int32_t end_id;
} m3o_model;

typedef struct {
  uint16_t* h_body;    /* [B, H]  body output before the final norm (optional) */
  float* logits0;      /* [B, V0] semantic logits ([B, 1 + V0] with the end
                          token, column 0) (optional)                         */
  float* zgap;         /* [B, 8]  best - second-best z per draw (optional)    */
} m3o_frame_trace;

/* The frame's parts, as m3o_decode_frame runs them (stage checks call them
   on the inputs a stage was given): one layer with the identity attention
   stub, in place on h [B, Hd]; depth step j's input from u and the codes
   [B, 8]; the next frame's input from the codes. */
void m3o_layer_stub(const m3o_layer* L, uint16_t* h, int B, int Hd, int n_heads, int n_kv,
                    int hd, int F, float eps);
/* the same layer with decode attention at position pos over the caches kc,
   vc ([B][n_kv][max_pos][hd]; slot pos is written) */
void m3o_layer_attn(const m3o_layer* L, uint16_t* h, int B, int Hd, int n_heads, int n_kv, int hd,
                    int F, float eps, const float* rope, uint16_t* kc, uint16_t* vc, int max_pos,
                    int pos);
void m3o_step_input(const m3o_model* m, int j, const int32_t* codes, const uint16_t* u, int B,
                    uint16_t* hd);
void m3o_feedback(const m3o_model* m, const int32_t* codes, int B, uint16_t* x_next);

/* codes[b*8 + 0] = absolute semantic id; codes[b*8 + j] = code j in [0,1024).
   x_next = bf16( (E_tok[c0] + sum_j A_j[c_j]) * 8^-1/2 ). */
void m3o_decode_frame(const m3o_model* m, const uint16_t* x_in, int B,
                      uint64_t seed, uint32_t frame, float temperature,
                      int32_t* codes, uint16_t* x_next, m3o_frame_trace* tr);

int m3o_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
