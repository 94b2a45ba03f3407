/*
 * m3.h -- C ABI of libm3: the per-frame autoregressive decode hot path of a
 * MiniMax-Music-3-style audio LM (Qwen3-shaped body + RVQ depth decoder) on
 * one AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory (packed weights, activations, outputs, workspaces); the library
 *    never allocates device memory on these paths.
 *  - bf16 values are passed as uint16_t bit patterns; fp32 as float.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream).  Results are valid once the stream
 *    reaches them.
 *  - Arguments are validated on the host BEFORE anything is launched; on a
 *    refusal the call returns a negative m3_status and enqueues nothing.
 *    Unsupported shapes are refused, never mis-computed (TensorFold PR #987,
 *    "Kernel contract": shapes within the bound, unsupported edges refused).
 *    A HIP launch error is reported as M3_ERR_HIP.
 *  - Determinism: identical inputs give byte-identical outputs; within one
 *    call, batch row b's result never depends on the other rows.
 *
 * Weight formats (TensorFold PR #987, precision list): bf16; int8 with one
 * fp32 scale per output row (body and lm_head); int8 with one fp32 scale per
 * group of 128 along K (depth decoder and its heads); quantised on the GPU
 * at load by m3_pack.
 */
#ifndef M3_H
#define M3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ----------------------------------------------------- */
typedef enum {
  M3_OK = 0,
  M3_ERR_NULL = -1,       /* a required pointer is NULL                      */
  M3_ERR_SHAPE = -2,      /* a size is outside the supported set             */
  M3_ERR_ALIGN = -3,      /* a pointer or leading dimension is misaligned    */
  M3_ERR_FORMAT = -4,     /* unknown weight format / epilogue / output type  */
  M3_ERR_WORKSPACE = -5,  /* workspace too small                             */
  M3_ERR_HIP = -6,        /* a HIP call failed (launch or graph error)       */
  M3_ERR_ALIAS = -7       /* an input overlaps an output it must not overlap */
} m3_status;

/* ---- enums ------------------------------------------------------------ */
enum { M3_BF16 = 0, M3_I8ROW = 1, M3_I8G128 = 2, M3_FP8ROW = 3 };  /* weight formats */
enum { M3_EPI_NONE = 0, M3_EPI_SWIGLU = 1, M3_EPI_RESIDUAL = 2 };
enum { M3_OUT_BF16 = 0, M3_OUT_F32 = 1 };
enum { M3_PACK_GLU_INTERLEAVE = 1 };

#define M3_MAX_B 64          /* lockstep rows per GEMV call                 */
#define M3_MAX_B_NORM_4K 16  /* rows when a 4096-wide norm is fused         */
#define M3_MAX_B_FRAME 16    /* rows per frame                              */
#define M3_MAX_B_SAMPLE 65535 /* rows per sampler call                      */
#define M3_MAX_SONGS_CFG 32767 /* songs (row pairs) per CFG draw call       */
#define M3_MAX_V_CFG 32768   /* columns per CFG draw call                   */
#define M3_MAX_M_PREFILL 65536 /* rows per prefill GEMM / RMSNorm call      */
#define M3_HEAD_DIM 128      /* attention head width (body and depth decoder) */
#define M3_MAX_POS 65536     /* cached positions per KV cache               */
#define M3_MAX_HEADS 256     /* query heads per attention call              */

const char* m3_status_str(int status);
/* library version string (host) */
const char* m3_version(void);

/* ---- packing (a load-time step) --------------------------------------- */
/* Packed layout, identical for all formats: the rows are cut into blocks of
 * 16; each block is a run of 1024-byte tiles along K, each tile holding 64
 * bytes of each of the 16 rows (32 bf16, or 64 int8 or fp8 values per row).  Byte
 * 16*l .. 16*l+15 of a tile belongs to row (l mod 16), K-bytes 16*(l/16) ..
 * 16*(l/16)+15 of the tile's 64-byte K-segment, so that one 16-byte load per
 * lane of a 64-lane wave reads the whole tile contiguously.  K is zero-padded
 * to a whole tile and N to a whole block.  int8 and fp8 blocks end with
 * their fp32 scales: i8row and fp8row: scale[r] for r = 0..15 (64 B, then
 * 64 B padding);
 * i8g128: scale[r][g] for the 16 rows and every group g of 128 along K
 * (16 x K/128 floats, rounded up to 128 B).  int8 codes are two's-complement
 * bytes in [-127, 127].  A packed matrix must be smaller than 2 GiB.
 *
 * Quantisation (int8): scale = absmax / 127 as one fp32 division; q is the
 * nearest integer of W/scale (ties to even), clamped to [-127, 127]; an
 * all-zero row or group gets scale 0.  Weights must be finite.
 *
 * Quantisation (fp8row, OCP FP8 E4M3: sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, exponent 0 = subnormals m * 2^-9, no infinity, largest
 * finite 448; the pages list fp8 weight-only only as a result on another
 * stack, diffusers issue #14486 and MiniMax-Music3 issue #2): scale =
 * absmax / 448 as one fp32 division per row; the code is the E4M3 value
 * nearest W/scale (ties to the even mantissa), saturated to +-448; an
 * all-zero row gets scale 0 and codes 0.
 *
 * flags & M3_PACK_GLU_INTERLEAVE: W is a stacked [gate; up] matrix [2F, K];
 * packed row 2i is gate row i and row 2i+1 is up row i, so one GEMV with the
 * SwiGLU epilogue produces both halves of each pair (TensorFold PR #987, "What
 * it adds": a gate and an up row whose SwiGLU the GEMV writes).  N = 2F.
 *
 * Sizes: bf16 K % 8 == 0; i8row, fp8row K % 16 == 0; i8g128 K % 128 == 0; N >= 1.
 * W_bf16 is [N, K] row-major (leading dimension K); W and packed must be
 * 16-byte aligned.  packed must hold m3_packed_bytes(fmt, N, K, flags). */
size_t m3_packed_bytes(int fmt, int N, int K, int flags);   /* host only; 0 = refused */
int m3_pack(int fmt, const uint16_t* W_bf16, int N, int K, int flags, void* packed,
            void* stream);

/* ---- RMSNorm-fused skinny GEMV/GEMM ------------------------------------ */
/* y[b, n] = epi( sum_k W[n, k] * a[b, k] ), fp32 accumulation, where
 *   a = x                                         if gamma == NULL
 *   a[b, k] = bf16(x[b, k] * r_b * gamma[k]),  r_b = (mean_k x[b,k]^2 + eps)^-1/2
 * (fp32 norm, bf16 operand: TensorFold PR #987 precision list; the norm is
 * folded into the GEMV that reads it, as that page's next steps propose).
 *
 * Attention stub (stub_group > 0): x is the [B, *] output row of a fused QKV
 * GEMV and the operand is a[b, h*hd + d] = x[b, stub_voff + (h/stub_group)*hd + d]
 * with hd = 128: identity attention over one cached position (the softmax
 * over a single key is 1), each query head reading its KV group's value.
 *
 * Epilogues:
 *   M3_EPI_NONE      y = acc (fp32) or bf16(acc)
 *   M3_EPI_RESIDUAL  y = bf16(residual + bf16(acc)); residual may equal y
 *                    (in-place update of the residual stream); bf16 out only
 *   M3_EPI_SWIGLU    rows are interleaved gate/up pairs (M3_PACK_GLU_INTERLEAVE);
 *                    y[b, i] = bf16(silu(bf16(acc_gate)) * bf16(acc_up)) rounded
 *                    once; y has N/2 columns; bf16 out only
 *
 * Sizes: 1 <= B <= M3_MAX_B; with gamma, B * roundup(K, tile) <= 65536
 * (B <= 16 at K = 4096, B <= 32 at K = 2048); ldx >= K (stub: >= voff + K/group),
 * ldy >= N (N/2 for SwiGLU), ldr >= N; x, y, residual 16-byte aligned and ldx,
 * ldy, ldr multiples of 8.  x must not overlap y.  eps >= 0. */
int m3_rmsnorm_gemv(const void* packed_bf16, int N, int K,
                    const uint16_t* x, int B, int ldx,
                    const float* gamma, float eps, int stub_group, int stub_voff,
                    void* y, int ldy, int out_dtype,
                    int epi, const uint16_t* residual, int ldr, void* stream);
int m3_gemv_i8row(const void* packed_i8row, int N, int K,
                  const uint16_t* x, int B, int ldx,
                  const float* gamma, float eps, int stub_group, int stub_voff,
                  void* y, int ldy, int out_dtype,
                  int epi, const uint16_t* residual, int ldr, void* stream);
/* fp8row: W[n, k] = scale[n] * E4M3(code[n, k]); the codes are converted to
 * bf16 exactly (every E4M3 value is a bf16) and multiplied in fp32, as for
 * int8.  Same parameters and bounds as m3_rmsnorm_gemv. */
int m3_gemv_fp8row(const void* packed_fp8row, int N, int K,
                   const uint16_t* x, int B, int ldx,
                   const float* gamma, float eps, int stub_group, int stub_voff,
                   void* y, int ldy, int out_dtype,
                   int epi, const uint16_t* residual, int ldr, void* stream);
int m3_gemv_i8g128(const void* packed_i8g128, int N, int K,
                   const uint16_t* x, int B, int ldx,
                   const float* gamma, float eps, int stub_group, int stub_voff,
                   void* y, int ldy, int out_dtype,
                   int epi, const uint16_t* residual, int ldr, void* stream);

/* ---- sliced lm_head ------------------------------------------------------ */
/* logits[b, j] = fp32( sum_k Wslice[j, k] * a[b, k] ), a = RMSNorm(x; gamma).
 * packed_slice holds only the reachable vocab rows (packed with m3_pack from
 * the full matrix's rows [row0, row0 + n_rows)): reading only the sampleable
 * rows gives the same draw as masking all other rows to -inf (diffusers issue
 * #14486 item 3; "MiniMax Music 3, local", where the time went).  Each
 * logit's summation order depends only on K, never on n_rows, the batch or
 * the slice offset, so a slice reproduces the full matrix's logits bit for
 * bit.  fmt is M3_BF16, M3_I8ROW or M3_FP8ROW.  Sizes as m3_rmsnorm_gemv; ldl >= n_rows,
 * ldl % 4 == 0. */
int m3_lmhead_sliced(int fmt, const void* packed_slice, int n_rows, int K,
                     const uint16_t* x, int B, int ldx, const float* gamma, float eps,
                     float* logits, int ldl, void* stream);

/* ---- Gumbel-argmax sampler ----------------------------------------------- */
/* out[b] = id of argmax_j z[b, j],  z = fl32(l[b, j] * fl32(1/T)) + G  (two
 * roundings, no contraction), ties to the lowest index, NaN above every number
 * (first NaN wins), ids outside [valid_lo, valid_hi) at -inf when lo < hi
 * (the vocab mask of DiffSynth-Studio's MiniMax-Music3 stage 2).  A draw from
 * softmax(l/T) (diffusers issue #14486 item 3: Gumbel-argmax in place of
 * softmax + multinomial).
 * G = -log(-log(u)), u = (2*(w >> 9) + 1) * 2^-24, w = word (id & 3) of
 * Philox-4x32-10 (Salmon et al., SC'11) with key (seed lo, seed hi) and
 * counter (id >> 2, b, frame, draw); id is the ABSOLUTE vocab id
 * (index_base + j, or ids[j]).  log is a fixed sequence of IEEE fp32
 * operations (frexp split + atanh series), so the noise is bit-reproducible.
 * frame_dev (optional): the frame number is read from device memory (the
 * frame counter the frame driver advances on the GPU).
 * noise_override (optional, device [B, V], row stride V): used in place of G. */
typedef struct {
  uint64_t seed;
  uint32_t frame;
  const uint32_t* frame_dev;     /* device, optional                         */
  uint32_t draw;                 /* 0 = semantic, 1..7 = depth codebooks      */
  float temperature;             /* > 0                                       */
  int32_t index_base;            /* absolute id of column 0 when ids == NULL  */
  const int32_t* ids;            /* device, optional [V]: absolute ids        */
  int32_t valid_lo, valid_hi;    /* mask; lo == hi disables it                */
  const float* noise_override;   /* device, optional [B, V]                   */
} m3_sample_params;

/* workspace bytes m3_gumbel_argmax needs for (B, V) (host) */
size_t m3_gumbel_workspace_bytes(int B, int V);
/* 1 <= B <= M3_MAX_B_SAMPLE, 1 <= V <= 2^24, ldl >= V; logits, out, ids,
 * noise_override, frame_dev 4-byte aligned, workspace 16-byte aligned.
 * params is a HOST struct. */
int m3_gumbel_argmax(const float* logits, int B, int V, int ldl,
                     const m3_sample_params* params, int32_t* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* m3_gumbel_argmax without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The per-chunk winners go to a fixed
 * array inside the library of M3_NOALLOC_SCRATCH_BYTES per device, held
 * until the process ends; (B, V) whose m3_gumbel_workspace_bytes exceeds it
 * are refused with M3_ERR_WORKSPACE before anything runs.  Every call on one
 * device shares that array: calls that overlap in time on a device race, so
 * keep them on one stream or order them with events.  Each call writes every
 * entry it reads (nothing has to start at zero).  Arguments, results and the
 * other errors as m3_gumbel_argmax; M3_ERR_HIP if the array's device address
 * cannot be looked up.  It calls no allocating routine. */
#define M3_NOALLOC_SCRATCH_BYTES (1u << 20)
int m3_gumbel_argmax_noalloc(const float* logits, int B, int V, int ldl,
                             const m3_sample_params* params, int32_t* out, void* stream);

/* ---- the reference's draw: guidance, top-k, multinomial ------------------ */
/* DiffSynth-Studio MiniMax-Music3 stage 2: each song's conditional row c and
 * unconditional row u are combined as u + cfg_scale (c - u) (scale 1.5 there),
 * filtered to the top_k largest (50 there) and sampled from the softmax of the
 * survivors; TensorFold PR #987 "What it adds" draws this on the same Philox
 * counters.  Song s owns logits rows 2s (conditional) and 2s+1
 * (unconditional), row stride ldl.  Per song:
 *   g_j = u_j + fl32(cfg_scale * fl32(c_j - u_j)) (three fp32 operations, no
 *         contraction); masked ids (params' valid range) and NaN g take no part;
 *   the survivors are the top_k largest g, ties to the lower column (all of
 *         them when fewer remain);
 *   the draw is Gumbel-argmax over the survivors, z = fl32(g * fl32(1/T)) + G
 *         with G as in m3_gumbel_argmax but counter row word = s (one draw
 *         per song), ranked as there (NaN on top, ties to the lower column);
 *         Gumbel-argmax draws from exactly the survivors' softmax(g/T);
 *   out[2s] = out[2s+1] = the drawn absolute id (a song with nothing left
 *         draws column 0's id).
 * noise_override (optional, device [n_songs, V]) replaces G.  Sizes:
 * 1 <= n_songs <= M3_MAX_SONGS_CFG, 1 <= V <= M3_MAX_V_CFG, ldl >= V,
 * top_k >= 1, cfg_scale finite, T > 0; logits, out, ids, noise_override,
 * frame_dev 4-byte aligned; params is a HOST struct.  Needs no workspace.
 * Errors: M3_ERR_NULL, M3_ERR_SHAPE, M3_ERR_ALIGN before any launch;
 * M3_ERR_HIP if the launch fails. */
int m3_cfg_topk_draw(const float* logits, int n_songs, int V, int ldl, float cfg_scale,
                     int top_k, const m3_sample_params* params, int32_t* out, void* stream);

/* ---- prompt prefill --------------------------------------------------------- */
/* A prompt of about 300 tokens for each of the two CFG rows ("MiniMax Music 3,
 * local"; TensorFold PR #987: 300 tokens a CFG row) runs every body matrix on
 * 600 rows at once: a dense contraction on the matrix cores.
 *
 * m3_rmsnorm_rows: a[m, k] = bf16((x[m, k] * r_m) * gamma[k]) with
 * r_m = 1 / sqrt(mean_k x[m, k]^2 + eps) in fp32 (the GEMV prologue's
 * arithmetic).  1 <= M <= M3_MAX_M_PREFILL; K % 8 == 0; ldx, lda >= K and
 * multiples of 8; x, a, gamma 16-byte aligned; x must not overlap a.
 *
 * m3_prefill_gemm: y[m, n] = epi( sum_k W[n, k] * a[m, k] ), fp32 accumulation
 * on v_mfma_f32_16x16x32_bf16, W packed bf16 by m3_pack (gate/up interleaved
 * for M3_EPI_SWIGLU).  Epilogues and outputs as m3_rmsnorm_gemv (SwiGLU and
 * residual write bf16; the residual may be y itself).  1 <= M <=
 * M3_MAX_M_PREFILL; N >= 1 (even for SwiGLU); K % 64 == 0; lda >= K, a
 * multiple of 8; ldy >= N (N/2 for SwiGLU); ldr >= N; the packed W and
 * the span of a ((M - 1) lda + K elements) each under 2 GiB; W, a, y 16-byte
 * aligned; a must not overlap y.  Errors: M3_ERR_NULL, M3_ERR_SHAPE,
 * M3_ERR_ALIGN, M3_ERR_FORMAT, M3_ERR_ALIAS before any launch; M3_ERR_HIP if
 * the launch fails. */
int m3_rmsnorm_rows(const uint16_t* x, int M, int K, int ldx, const float* gamma, float eps,
                    uint16_t* a, int lda, void* stream);
int m3_prefill_gemm(const void* packed_bf16, int N, int K, const uint16_t* a, int M, int lda,
                    void* y, int ldy, int out_dtype, int epi, const uint16_t* residual, int ldr,
                    void* stream);

/* ---- decode attention -------------------------------------------------------- */
/* Attention of each batch row's new query over its cached positions, in place of
 * the identity stub ("MiniMax Music 3, local" and TensorFold PR #987 list per-head
 * q/k norm + RoPE, split-key decode attention with a merge, and the depth
 * decoder's attention over its codebook positions; fp32 norms, RoPE, softmax and
 * sums over bf16 activations).  Head width 128 (M3_HEAD_DIM).  KV caches are bf16
 * [B][n_kv][max_pos][128], caller-allocated.  Query head h reads KV head
 * h / (n_q / n_kv); n_q / n_kv must be 1, 2, 4 or 8.
 *
 * m3_rope_table: table[(p * 64 + i) * 2 + {0, 1}] = fl32(cos / sin(p * theta^(-i/64)))
 * for p < max_pos, i < 64, angle and trig in float64 (Qwen3: theta = 1e6).
 * table: device, 16-byte aligned, max_pos * 128 floats.
 *
 * m3_qk_norm_rope: for every row b of qkv (q heads at columns h*128, then the
 * n_kv k heads, then the n_kv v heads): per head RMSNorm over its 128 values,
 * x' = bf16((x * r) * gamma) with r = 1 / sqrt(mean x^2 + eps) in fp32 (q_gamma
 * for q heads, k_gamma for k heads; 128 floats each), then the rotation of the
 * pairs (i, i + 64) by the table's angle at position pos:
 *   y_i = bf16(x'_i c - x'_{i+64} s),  y_{i+64} = bf16(x'_{i+64} c + x'_i s).
 * q goes to q_out [B, ldq]; k and the unnormed v go to the caches at position pos.
 * rope is a table from m3_rope_table with more than pos positions.
 * 1 <= B <= M3_MAX_B; 0 <= pos < max_pos <= M3_MAX_POS; ldqkv >= (n_q + 2 n_kv)
 * * 128, ldq >= n_q * 128, both multiples of 8; qkv, q_out, caches, rope 16-byte
 * aligned; no two of qkv, q_out, k_cache, v_cache overlap.
 *
 * m3_decode_attention: out[b, h*128 + d] = bf16( sum_{t<T} p_t v[b][h/g][t][d] ),
 * p = softmax_t( q[b,h] . k[b][h/g][t] / sqrt(128) ), fp32 sums and softmax
 * (base-2 exponentials with the scale folded in).  Positions are split into
 * chunks of 128 (64 when B * n_kv * ceil(T / 128) < 256); with more than one
 * chunk the partial softmax states go to the workspace and a second launch
 * merges them in chunk order.  The workspace (m3_attention_workspace_bytes(B,
 * n_q, n_kv, T) bytes, 0 for a single chunk; device, 16-byte aligned,
 * caller-owned, no contents kept between calls) may be shared by calls that
 * do not overlap in time.  1 <= T <= max_pos; ldq, ldo >= n_q *
 * 128, multiples of 8; q, caches, out 16-byte aligned; out and the workspace
 * overlap nothing else.
 *
 * Errors (all three calls): M3_ERR_NULL, M3_ERR_SHAPE, M3_ERR_ALIGN,
 * M3_ERR_WORKSPACE, M3_ERR_ALIAS before any launch; M3_ERR_HIP if a launch fails. */
int m3_rope_table(float* table, int max_pos, int head_dim, float theta, void* stream);
int m3_qk_norm_rope(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv, int head_dim,
                    const float* q_gamma, const float* k_gamma, float eps, const float* rope,
                    int pos, uint16_t* q_out, int ldq, uint16_t* k_cache, uint16_t* v_cache,
                    int max_pos, void* stream);
size_t m3_attention_workspace_bytes(int B, int n_q, int n_kv, int T);
int m3_decode_attention(const uint16_t* q, int B, int ldq, int n_q, int n_kv, int head_dim,
                        const uint16_t* k_cache, const uint16_t* v_cache, int max_pos, int T,
                        uint16_t* out, int ldo, void* workspace, size_t workspace_bytes,
                        void* stream);
/* One decode step's attention ("MiniMax Music 3, local" and TensorFold PR
 * #987, kernel list: q/k norm + RoPE, split-key decode attention with a
 * merge): m3_qk_norm_rope at pos (the caches' slot pos written) followed by
 * m3_decode_attention over T = pos + 1 positions, in one launch plus the
 * merge, with the same results and no q buffer.  Arguments as those two
 * calls (workspace: m3_attention_workspace_bytes(B, n_q, n_kv, pos + 1)
 * bytes); qkv, out, the caches and the workspace overlap nothing else.
 * Errors as m3_decode_attention. */
int m3_decode_attention_step(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                             int head_dim, const float* q_gamma, const float* k_gamma, float eps,
                             const float* rope, int pos, uint16_t* k_cache, uint16_t* v_cache,
                             int max_pos, uint16_t* out, int ldo, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- the prompt's attention ------------------------------------------------- */
/* The prompt's rows through the same steps as one decode row, all positions at
 * once: S sequences (the CFG rows) of P prompt positions, rows ordered [s][t],
 * row (s, t) at position pos_base + t of sequence s's cache.
 *
 * m3_prefill_qk_norm_rope: as m3_qk_norm_rope for every row at its own
 * position; k and v of row (s, t) go to slot pos_base + t of cache s ([S][n_kv]
 * [max_pos][128]).  The caches then hold the prompt for decode attention.
 *
 * m3_prefill_attention: causal attention, row (s, t) over positions 0 ..
 * pos_base + t of cache s: fp32 scores of the bf16 q and keys, scaled to
 * base 2, a softmax with a running maximum and fp32 P.V over chunks of 64
 * keys, out = bf16(P.V / sum), one workgroup per block of rows.  No workspace:
 * m3_prefill_attention_workspace_bytes returns 0 and the workspace arguments
 * are ignored (they may be NULL, 0).
 *
 * 1 <= S <= M3_MAX_B; S * P <= M3_MAX_M_PREFILL; 0 <= pos_base, pos_base + P
 * <= max_pos <= M3_MAX_POS; the other sizes, alignment and aliasing rules and
 * the errors as for the decode calls. */
int m3_prefill_qk_norm_rope(const uint16_t* qkv, int S, int P, int ldqkv, int n_q, int n_kv,
                            int head_dim, const float* q_gamma, const float* k_gamma, float eps,
                            const float* rope, int pos_base, uint16_t* q_out, int ldq,
                            uint16_t* k_cache, uint16_t* v_cache, int max_pos, void* stream);
size_t m3_prefill_attention_workspace_bytes(int S, int P, int n_q, int n_kv, int pos_base);
int m3_prefill_attention(const uint16_t* q, int S, int P, int ldq, int n_q, int n_kv, int head_dim,
                         const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                         int pos_base, uint16_t* out, int ldo, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---- one decode frame ------------------------------------------------------ */
typedef struct {
  int hidden, n_layers, n_heads, n_kv_heads, head_dim, ffn;
  int vocab_base, n_slice;        /* reachable ids [vocab_base, vocab_base+n_slice) */
  int d_hidden, d_layers, d_heads, d_head_dim, d_ffn;
  int n_codebooks, code_vocab;
  int fmt_body, fmt_lm, fmt_depth;
  float eps, temperature;
  uint64_t seed;
  /* The frame's draws.  top_k == 0: one Gumbel-argmax draw per row (the
   * benchmark configuration).  top_k > 0: the reference's draw
   * (DiffSynth-Studio MiniMax-Music3 stage 2: guidance u + cfg_scale (c - u)
   * over each (conditional, unconditional) row pair, top-k, multinomial), as
   * m3_cfg_topk_draw: rows 2s and 2s+1 form song s (B even), every one of the
   * 8 draws is made once per song and both rows take it.  Eager and graph
   * frames only; n_slice and code_vocab <= M3_MAX_V_CFG. */
  float cfg_scale;
  int top_k;
  /* Attention.  0: the identity stub (one cached position, softmax over one
   * key is 1; the benchmark configuration).  1: decode attention over KV
   * caches kept in the frame state: in every body layer, q/k RMSNorm with the
   * layer's q_norm / k_norm, RoPE (base 1e6) at position pos0 + frame counter
   * (read on the GPU, so graph replays advance it), the k/v cache write and
   * softmax attention over the positions up to it, as m3_qk_norm_rope and
   * m3_decode_attention; in the depth decoder, the same over the frame's
   * codebook positions (position j - 1 at step j, a cache per layer reused
   * every frame).  max_pos: cached positions per body layer (1 ..
   * M3_MAX_POS); 0 <= pos0 < max_pos.  A frame whose position reaches max_pos
   * is refused on the GPU: it rewrites slot max_pos - 1, attends over max_pos
   * positions and sets the state's err word to M3_ERR_ATTN_FULL (a
   * persistent frame then ends its waits, as below). */
  int attention;
  int max_pos;
  int pos0;
  /* The end of a song (DiffSynth-Studio MiniMax-Music3 stage 2: the semantic
   * draw is masked to the audio codes and the end token, and generation
   * stops once the end token is drawn).  end_id < 0: no end token, the draw
   * is over the n_slice codes (the benchmark configuration).  0 <= end_id <
   * vocab_base: the lm_head holds n_slice + 1 rows, row 0 the end token's
   * and row 1 + i code i's, and the draw takes the end token like any other
   * id (Gumbel noise keyed by end_id; an exact tie goes to the lower id,
   * i.e. to it).  A row that draws it gets end_id as its semantic code; its
   * depth step 1 input and frame embedding use code 0's rows (the frame is
   * still computed, in lockstep with the other rows), and the state's stop
   * word of the row becomes the frame number + 1 the first time.  The host
   * reads the stop words (or the end token in the ring) every 16 frames
   * (TensorFold PR #987, frame pipelining). */
  int end_id;
} m3_config;

#define M3_ERR_ATTN_FULL 2u  /* state err word: the frame position reached max_pos */

typedef struct {
  const void* qkv;        /* packed [nq + 2 nkv, hidden]              */
  const void* o;          /* packed [hidden, nq]                      */
  const void* gate_up;    /* packed, GLU-interleaved [2 ffn, hidden]  */
  const void* down;       /* packed [hidden, ffn]                     */
  const float* attn_norm; /* [hidden] */
  const float* ffn_norm;  /* [hidden] */
  const float* q_norm;    /* [head_dim] per-head q RMSNorm (attention = 1 only) */
  const float* k_norm;    /* [head_dim] per-head k RMSNorm (attention = 1 only) */
} m3_layer_weights;

typedef struct {
  m3_config cfg;
  const m3_layer_weights* layers;     /* host array [n_layers]                   */
  const float* final_norm;            /* [hidden]                                */
  const void* lm_head;                /* packed slice [n_slice, hidden] (fmt_lm);
                                         [1 + n_slice, hidden] with the end token's
                                         row first when cfg.end_id >= 0          */
  const void* p_in;                   /* packed [d_hidden, hidden] (fmt_depth)   */
  const uint16_t* emb1;               /* bf16 [n_slice, d_hidden]                */
  const uint16_t* const* emb;         /* host array [n_codebooks-2] of [code_vocab, d_hidden] */
  const m3_layer_weights* d_layers_w; /* host array [d_layers]                   */
  const float* d_final_norm;          /* [d_hidden]                              */
  const void* const* heads;           /* host array [n_codebooks-1], packed [code_vocab, d_hidden] */
  const uint16_t* tok_emb_audio;      /* bf16 [n_slice, hidden]: embed_tokens rows of the codes */
  const uint16_t* const* audio_emb;   /* host array [n_codebooks-1] of [code_vocab, hidden] */
} m3_model;

/* Device buffers inside the frame state (byte offsets from its base).
 * Every GEMV output of every body layer, and of every depth-decoder layer of
 * every codebook step, has a slot of its own, as do each depth step's input
 * and each depth head's logits: nothing is written twice within a frame, and
 * each operation of a frame can be checked on its own from the input it was
 * given (TensorFold PR #987, summary: parity at every stage, teacher-forced).
 * Slots are plain bf16 after an eager or graph frame; a persistent frame
 * writes the tagged buffers instead (and a plain copy of the body output).
 * Shapes: L = n_layers, S = n_codebooks - 1 depth steps, DL = d_layers. */
typedef struct {
  size_t x;        /* bf16 [B, hidden]   frame input; overwritten by x_next    */
  size_t h;        /* bf16 [L][B, hidden] residual stream after each body layer;
                      the last slot is the body output                         */
  size_t qkv;      /* bf16 [L][B, nq+2nkv] each layer's QKV output              */
  size_t mlp;      /* bf16 [L][B, ffn]   each layer's SwiGLU output            */
  size_t logits;   /* f32  [B, n_slice (+1 with the end token, column 0)]
                      semantic logits of the last frame                        */
  size_t u;        /* bf16 [B, d_hidden] depth-decoder input projection        */
  size_t hd;       /* bf16 [S][DL+1][B, d_hidden]: for step j (codebook j = 1..7,
                      slot j-1) its input bf16(u + Emb_j[c]) in slot 0 and the
                      residual stream after depth layer l in slot l+1          */
  size_t dqkv;     /* bf16 [S][DL][B, 3 d_hidden]                              */
  size_t dmlp;     /* bf16 [S][DL][B, d_ffn]                                   */
  size_t dlogits;  /* f32  [S][B, code_vocab] each step's head logits          */
  size_t ring;     /* i32  [16, B, 8]    codes of the last 16 frames           */
  size_t frame;    /* u32  frame counter (advanced on the GPU)                 */
  size_t part_sem; /* per-row-block winners of the semantic draw               */
  size_t part_dep; /* [S]: per-row-block winners of each depth step's draw     */
  size_t flags;    /* u32  [256] per-workgroup progress of the persistent frame */
  size_t err;      /* u32  nonzero: a persistent frame gave up waiting          */
  size_t seq;      /* u32  the persistent frame's epoch (launch counter)       */
  size_t phases;   /* the persistent frame's phase table                       */
  size_t th, tqkv, tmlp, tu, thd, tdqkv, tdmlp;
                   /* u32 words (bf16 value | 16-bit producer tag): the
                      persistent frame's streams, shaped as h, qkv, mlp, u,
                      hd, dqkv, dmlp above                                     */
  size_t th2, thd2; /* u32 words [L][B, hidden], [S][DL][B, d_hidden]: the
                      persistent frame's streams after O, shaped as ho, hdo   */
  size_t ho, hdo;  /* bf16 [L][B, hidden], [S][DL][B, d_hidden]: the residual
                      stream after O (+ residual) of each layer                 */
  /* attention = 1 only (zero-sized otherwise): */
  size_t rope;     /* f32  [max(max_pos, 8), 64, 2] RoPE table                 */
  size_t aq;       /* bf16 [B, max(nq, d_hidden)] reserved scratch            */
  size_t ao;       /* bf16 [L][B, nq]    each body layer's attention output    */
  size_t dao;      /* bf16 [S][DL][B, d_hidden] each depth layer's attention output */
  size_t kcache, vcache;   /* bf16 [n_layers][B][n_kv][max_pos][128]          */
  size_t dkcache, dvcache; /* bf16 [d_layers][B][d_heads][8][128]             */
  size_t attn_ws;  /* m3_decode_attention's workspace at T = max_pos           */
  size_t tao, tdao; /* u32 words [L][B, nq], [S][DL][B, d_hidden]: the
                      persistent frame's attention outputs, shaped as ao, dao  */
  size_t trec;     /* [L][B][n_kv][chunks][nq / n_kv][2 + 128] 64-bit words (fp32
                      value | 16-bit producer tag << 32): the persistent frame's
                      chunk records of each body layer's attention (zero-sized
                      when one chunk covers max_pos)                          */
  size_t stop;     /* int32 [B]: 0, or 1 + the frame that drew the end token    */
  size_t kpart;    /* f32 wave partial sums of the eager and graph frames' GEMVs
                      split along K (down projections whose B-row operand does
                      not fit LDS: B >= 7 in the body at K = 12288); scratch   */
  size_t kcnt;     /* u32 counters of those GEMVs' row-block groups; zero
                      between launches (set by m3_frame_state_init, left zero by
                      every launch)                                            */
  size_t total;
} m3_frame_layout;

/* Algorithmic weight bytes one frame streams: every body matrix once, the
 * lm_head slice once (with the end token's row when end_id >= 0), the depth
 * input projection once, the depth layers and
 * one head per codebook step (7 steps), plus the fp32 gammas of every norm
 * application.  bf16: 2NK; i8row: NK + 4N; i8g128: NK + 4N*K/128.
 * (TensorFold PR #987, frame anatomy: the engine accounts for each frame's
 * weight traffic.) */
uint64_t m3_frame_weight_bytes(const m3_config* cfg /* host */);
/* layout of the caller-allocated frame state; 0 / M3_ERR_* on refusal */
int m3_frame_layout_get(const m3_config* cfg /* host */, int B, m3_frame_layout* out /* host */);
size_t m3_frame_workspace_bytes(const m3_config* cfg /* host */, int B);
/* Zero the frame state, copy x0 (device bf16 [B, hidden]) into its input and
 * set the frame counter to frame0. */
int m3_frame_state_init(const m3_config* cfg, int B, void* state, const uint16_t* x0,
                        uint32_t frame0, void* stream);
/* Enqueue one frame: body (per layer: norm+QKV, stub+O+residual, norm+gate/up
 * +SwiGLU, down+residual; with attention = 1 the stub is q/k norm + RoPE, the
 * cache write and attention at the frame's position, then O+residual) -> final
 * norm + sliced lm_head -> draw 0 -> depth
 * input projection -> 7 x (embedding of the previous code, depth layers, final
 * norm + head_j, draw j) -> feedback x' = bf16((E_tok[c0] + sum_j A_j[c_j]) *
 * 8^-1/2) into the state's input, codes into `codes` (device [B, 8]: absolute
 * semantic id, then codes 1..7) and into the 16-frame ring, frame counter + 1
 * on the GPU (DiffSynth-Studio MiniMax-Music3 stage 2; TensorFold PR #987:
 * position and count advance on the GPU, the host reads the drawn tokens
 * every 16 frames).  1 <= B <= M3_MAX_B_FRAME.  bytes_read (host, optional)
 * receives m3_frame_weight_bytes. */
int m3_decode_frame_weights(const m3_model* model /* host */, void* state, int B,
                            int32_t* codes, uint64_t* bytes_read, void* stream);

/* HIP-graph form of the frame: capture the launches of one frame once and
 * replay them; every replay is a new frame (the counter lives on the GPU).
 * The captured graph keeps the model's and the state's device addresses. */
int m3_frame_graph_create(const m3_model* model, void* state, int B, int32_t* codes,
                          void* stream, void** graph_out /* host */);
int m3_frame_graph_launch(void* graph, void* stream);
int m3_frame_graph_destroy(void* graph);
/* The RVQ depth decoder of a frame alone, as a graph for
 * m3_frame_graph_launch / _destroy (DiffSynth-Studio MiniMax-Music3 stage 2:
 * the depth input projection, then 7 codebook steps of the depth layers, each
 * with its head and draw, then the feedback): the same launches as the
 * frame's from the depth input projection on.  It reads the body output and
 * the semantic draw that the state holds from its last whole frame (run one
 * first; until then they are zeros); each replay writes codes 1..7, the
 * 16-frame ring, the fed-back input and the frame counter like a whole frame
 * (the semantic code in `codes` is the last whole frame's).  For timing the
 * depth decoder on its own. */
int m3_depth_graph_create(const m3_model* model, void* state, int B, int32_t* codes,
                          void* stream, void** graph_out /* host */);

/* Persistent form of the frame: the same steps, with the same results, run as
 * ONE cooperative launch per frame.  One workgroup per compute unit walks the
 * frame's steps in order (GEMVs and, with attention = 1, each layer's
 * attention: q/k norm + RoPE, the cache write, the chunks' partial softmax
 * and their merge as one step, with the decode attention calls' chunking and
 * arithmetic; G = n_q / n_kv of 1, 2 or 4); each workgroup requests the first weight tiles of
 * the next GEMV before it waits for the previous GEMV's outputs, so HBM keeps
 * streaming across the ~270 dependencies of a frame (TensorFold PR #987: one submission per frame;
 * "MiniMax Music 3, local": the AR stages are bound by memory bandwidth).
 * create records the frame into the state's phase table (it synchronises
 * `stream` once); launch enqueues one frame; the handle keeps the model's and
 * the state's device addresses.  Every wait inside the launch is bounded: if
 * one gives up (the launch could not make progress), the state's err word
 * becomes nonzero, the launch ends early and that frame's outputs are invalid;
 * while the word is nonzero, launches on the state return at once and compute
 * nothing.  m3_frame_persistent_create clears it: each create starts a new
 * epoch of the tags (below), so nothing a launch that gave up left behind is
 * taken for an operand later.
 * Inside the launch the intermediate streams (body and depth residuals, QKV,
 * MLP, depth input, attention outputs) are the state's tagged buffers: 32-bit words holding the
 * bf16 value and the tag of the step that wrote it; a step waits for its
 * operand by reading it until the tags are the ones its producer writes (one
 * store and one load per dependency, no barrier).  x, h, logits, codes, the
 * ring and the frame counter are updated exactly as by the other paths, with
 * the same bytes.  Supported: bf16, int8-row or fp8-row body with the same lm_head
 * format and an int8-g128 depth decoder (else M3_ERR_FORMAT), every GEMV
 * operand staged in LDS (at the full model: B <= 6; else M3_ERR_SHAPE), the
 * guided draw (top_k > 0) over at most 18432 columns (its draw phases: the
 * draw kernel's search with one 512-thread workgroup per song), vocab
 * slice and code vocabulary below 65536.  The frame state must have been
 * initialised with m3_frame_state_init; eager, graph and persistent frames may
 * be interleaved on one state.  The launch fails with M3_ERR_HIP if the device
 * cannot hold one workgroup per compute unit at once. */
int m3_frame_persistent_create(const m3_model* model, void* state, int B, int32_t* codes,
                               void* stream, void** handle_out /* host */);
int m3_frame_persistent_launch(void* handle, void* stream);
int m3_frame_persistent_destroy(void* handle);

/* Phase clock of a persistent frame (profiling; off by default).  With a
 * device buffer attached, every later launch on the handle has thread 0 of
 * each workgroup write the GPU's constant-rate real-time counter
 * (s_memrealtime) at three points of every phase i: entry (slot 0), its
 * operand staged (slot 1; the frame end: every workgroup's flag seen) and
 * the phase's end (slot 2), to clk[(slot * n_phases + i) * n_workgroups +
 * wg]; a workgroup with no rows in a phase writes no slot 1 there.  clk ==
 * NULL detaches the buffer.  clk_bytes >= m3_frame_persistent_clock_bytes;
 * the buffer is caller-owned, 8-byte aligned.  n_phases and n_workgroups
 * (host, optional) receive the table's dimensions.  Values are unchanged
 * with the clock attached; the frame takes slightly longer. */
size_t m3_frame_persistent_clock_bytes(void* handle);
int m3_frame_persistent_clock(void* handle, uint64_t* clk, size_t clk_bytes, int* n_phases,
                              int* n_workgroups);

/* The persistent frame's steps as records of the memory each step reads and
 * writes (host only: nothing is launched and no memory is touched; the state
 * and model pointers only fix addresses).  Record i is step i of the
 * persistent launch (a GEMV, an attention step, a guided draw, which waits
 * for every workgroup to finish the logits step before it, or the frame end,
 * which runs after every workgroup has finished every other step); a region is `rows`
 * rows of bytes [base + r stride + c0, base + r stride + c1), with the step
 * that produced what is read (-1: written before the launch, or by an
 * earlier step of the frame for the frame end; for a draw, the step before
 * it; for an attention step's
 * cache reads, by the step itself or by the same layer's attention at the
 * frame's earlier codebook steps) and whether its words carry the producer's
 * tag.  A consumer waits for the tags of its producer, so the ordering this
 * rests on can be checked from the table: every tagged input is written by
 * its producer, earlier, and no byte is written twice in a frame.  Returns
 * the number of steps, or M3_ERR_* (M3_ERR_WORKSPACE: out has fewer than
 * that many records; out may be NULL to count; M3_ERR_FORMAT: the frame has
 * no persistent form). */
#define M3_PHASE_MAX_REGIONS 4
enum { M3_PHASE_GEMV = 0, M3_PHASE_FRAME_END = 1, M3_PHASE_ATTENTION = 2, M3_PHASE_DRAW = 3 };
typedef struct {
  uint64_t base, stride;
  int32_t rows;
  uint32_t c0, c1;
  int32_t producer;
  int32_t tagged;
  int32_t pad;
} m3_phase_region;
typedef struct {
  int32_t kind;
  int32_t n_in, n_out;
  int32_t pad;
  m3_phase_region in[M3_PHASE_MAX_REGIONS];
  m3_phase_region out[M3_PHASE_MAX_REGIONS];
} m3_phase_record;
int m3_frame_phase_table(const m3_model* model, void* state, int B, int32_t* codes,
                         m3_phase_record* out /* host */, int max_records);

/* ---- measurement ------------------------------------------------------------ */
/* A plain streaming read of `bytes` at buf (16-byte aligned, a multiple of 16,
 * below 2 GiB): `workgroups` (1..4096) workgroups of 512 lanes read it with 16-byte
 * buffer loads, the GEMVs' weight-tile loads (nontemporal: their cache
 * policy for weights read once per frame; 0: the default policy), and each
 * writes one word of what it read to sink[workgroup] (device, 4-byte
 * aligned).  The read rate this reaches on the device is the ceiling the
 * decode's weight stream is compared with, next to the HBM spec peak.
 * Errors: M3_ERR_NULL, M3_ERR_SHAPE, M3_ERR_ALIGN before the launch; the HIP
 * launch status otherwise. */
int m3_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, int nontemporal,
                   void* stream);

#ifdef __cplusplus
}
#endif
#endif /* M3_H */
