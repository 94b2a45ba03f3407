// m3_internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/m3.h"
#include "m3_sampling.h"

namespace m3 {

// ---- packed weight layout (see m3.h, "Packed layout") ----------------------
constexpr int kTileBytes = 1024;   // 16 rows x 64 bytes
constexpr int kRowsPerBlock = 16;

__host__ __device__ inline int tile_k(int fmt) { return fmt == M3_BF16 ? 32 : 64; }
__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }
__host__ __device__ inline int k_pad(int fmt, int K) { return round_up(K, tile_k(fmt)); }
__host__ __device__ inline int n_tiles(int fmt, int K) { return k_pad(fmt, K) / tile_k(fmt); }
__host__ __device__ inline int n_blocks(int N) { return (N + kRowsPerBlock - 1) / kRowsPerBlock; }
__host__ __device__ inline int scale_bytes(int fmt, int K) {
  return (fmt == M3_I8ROW || fmt == M3_FP8ROW) ? 128
                                               : (fmt == M3_I8G128 ? round_up((K / 128) * 64, 128) : 0);
}
__host__ __device__ inline size_t block_bytes(int fmt, int K) {
  return (size_t)n_tiles(fmt, K) * kTileBytes + scale_bytes(fmt, K);
}

// ---- GEMV launch description -------------------------------------------------
// Gumbel sampling epilogue of a logits GEMV (fp32 out): besides the logits,
// every row block writes the best (z, column) of its 16 rows for each batch
// row to part[b * nblocks + block].
struct SampleEpi {
  uint64_t seed;
  const uint32_t* frame;        // device frame counter
  uint32_t draw;
  float temperature;
  int32_t index_base;           // absolute id of output row 0
  int32_t valid_lo, valid_hi;   // lo == hi: no mask
  Best* part;
  int32_t end_id;               // >= 0: output row 0 is this id (the end token; never masked)
};

// Gather prologue of the first GEMV of a depth-decoder step: the operand row
// b is bf16(u[b] + emb[c_b]) with c_b = index_base + argmax of part[b][*]
// (the previous draw) minus code_base (0 if out of range).  Workgroup 0 also
// writes the rows to out (the step's residual stream) and the drawn absolute
// id to codes[b * 8 + code_col].
struct GatherPro {
  const uint16_t* u;
  const uint16_t* emb;
  const Best* part;
  int nparts;
  int32_t index_base, code_base, n_codes;
  int32_t* codes;
  int code_col;
  uint16_t* out;
  int32_t end_id;               // >= 0: part's column 0 is this id (the end token)
};

struct GemvDesc {
  int fmt;
  const void* w;
  int N, K;
  const uint16_t* x;
  int ldx, B;
  const float* gamma;
  float eps;
  int stub_group, stub_voff;
  void* y;
  int ldy, out_f32;
  int epi;
  const uint16_t* res;
  int ldr;
  const SampleEpi* sample = nullptr;
  const GatherPro* gather = nullptr;
  // persistent frame only: producing phase of x / residual / gather u /
  // gather partials (-1: plain buffer), tagged outputs
  int px = -1, pres = -1, pu = -1, ppart = -1, ytag = 0;
  // persistent frame only, scheduling (no effect on any value): rot = the
  // row block taken first (blocks in the order rot, rot + 1, ... mod the
  // count); follow = the block count of the phase before, whose workgroups
  // with one block fewer take this phase's blocks first (0: workgroup 0)
  int rot = 0, follow = 0;
  // one-launch frames only (no effect on any value): a GEMV without a fused
  // norm whose B-row operand does not fit LDS may run split along K (see
  // gemv.hip) with these: fp32 wave partials for kpart_blocks row blocks and
  // one counter per group of row blocks, zero between launches
  float* kpart = nullptr;
  uint32_t* kcnt = nullptr;
  int kpart_blocks = 0;
};

// Largest fused-norm activation block held in LDS (elements of B * K_pad).
constexpr int kMaxNormElems = 65536;

hipError_t launch_gemv(const GemvDesc& d, hipStream_t s);
// the split-K workspace for GEMVs of up to nblocks row blocks: partial bytes
// and group counters (GemvDesc::kpart, kcnt)
size_t gemv_split_part_bytes(int nblocks);
size_t gemv_split_counters(int nblocks);
// dynamic LDS bytes launch_gemv uses for (fmt, K, B, fused norm); > 160 KiB = unsupported
size_t gemv_smem_bytes(int fmt, int K, int B, bool has_gamma);
// set kernel attributes of every GEMV instantiation (before graph capture)
hipError_t gemv_prepare();
hipError_t launch_pack(int fmt, const uint16_t* W, int N, int K, int flags, void* packed,
                       hipStream_t s);

// ---- sampler -----------------------------------------------------------------
struct SampleDesc {
  const float* logits;
  int B, V, ldl;
  uint64_t seed;
  uint32_t frame;
  const uint32_t* frame_dev;
  uint32_t draw;
  float temperature;
  int32_t index_base;
  const int32_t* ids;
  int32_t valid_lo, valid_hi;
  const float* noise;
  int32_t* out;
  int out_stride;       // out[b * out_stride]
  void* ws;
};
size_t sample_ws_bytes(int B, int V);
hipError_t launch_sample(const SampleDesc& d, hipStream_t s);
// The allocation-free draw: a file-scope device array of this many bytes
// (each device holds its own copy) serves as the workspace; sample_scratch
// returns the current device's address of it (looked up once per device).
constexpr size_t kSampleScratchBytes = M3_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
hipError_t sample_scratch(void** ptr);

// CFG + top-k draw: one workgroup per song; rows 2s / 2s+1 are the song's
// conditional / unconditional logits; out[(2s) * out_stride] and
// out[(2s+1) * out_stride] receive its id.  V <= kCfgMaxV (32 keys per thread).
constexpr int kCfgMaxV = M3_MAX_V_CFG;
struct CfgDesc {
  const float* logits;
  int S, V, ldl;
  float scale;
  int top_k;
  uint64_t seed;
  uint32_t frame;
  const uint32_t* frame_dev;
  uint32_t draw;
  float temperature;
  int32_t index_base;
  const int32_t* ids;
  int32_t valid_lo, valid_hi;
  const float* noise;   // [S, V] or null
  int32_t* out;
  int out_stride;
  int vec4;             // logits rows 16-byte aligned (float4 loads)
  Best* part;           // non-null: write {0, column} to part[2s], part[2s+1] instead of ids
  int32_t end_id = -1;  // >= 0: column 0 is this id (the end token; never masked)
};
hipError_t launch_cfg_draw(const CfgDesc& d, hipStream_t s);

// ---- prompt prefill (prefill.hip) ---------------------------------------------
// Y[M, N] = epi(A[M, K] . W^T), W packed bf16 (m3_pack), K % 64 == 0.
struct PrefillDesc {
  const void* w;
  int N, K;
  const uint16_t* a;
  int M, lda;
  void* y;
  int ldy, out_f32, epi;
  const uint16_t* res;
  int ldr;
};
hipError_t launch_prefill_gemm(const PrefillDesc& d, hipStream_t s);
hipError_t launch_rmsnorm_rows(const uint16_t* x, int M, int K, int ldx, const float* gamma,
                               float eps, uint16_t* a, int lda, hipStream_t s);

// ---- decode attention (attention.hip) --------------------------------------------
int attn_chunk_size(int B, int n_kv, int T);
size_t attn_workspace_bytes(int B, int n_q, int n_kv, int T);
hipError_t launch_rope_table(float* t, int max_pos, int head_dim, double theta, hipStream_t s);
// frame_dev (optional, device): the position is pos0 + *frame_dev (held below
// max_pos; past it, err gets M3_ERR_ATTN_FULL) and T = position + 1.
// P > 1 (prompt rows): row r is position pos + r % P of cache sequence r / P
// and attends over T + r % P positions.
hipError_t launch_qk_norm_rope(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                               const float* q_gamma, const float* k_gamma, float eps,
                               const float* rope, int pos, uint16_t* q_out, int ldq,
                               uint16_t* k_cache, uint16_t* v_cache, int max_pos, hipStream_t s,
                               const uint32_t* frame_dev = nullptr, int pos0 = 0,
                               uint32_t* err = nullptr, int P = 1);
// the prompt's causal attention: S sequences of P rows, row (s, t) over
// positions 0 .. pos_base + t of cache s; no workspace
hipError_t launch_prompt_attention(const uint16_t* q, int S, int P, int ldq, int n_q, int n_kv,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                                   int pos_base, uint16_t* out, int ldo, hipStream_t s);
hipError_t launch_decode_attention(const uint16_t* q, int B, int ldq, int n_q, int n_kv,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                                   int T, uint16_t* out, int ldo, void* ws, hipStream_t s,
                                   const uint32_t* frame_dev = nullptr, int pos0 = 0, int P = 1);
// the two above in one launch (plus the merge), one position per row: the
// frame's attention steps (same results)
hipError_t launch_attention_fused(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                                  const float* q_gamma, const float* k_gamma, float eps,
                                  const float* rope, int pos, uint16_t* k_cache,
                                  uint16_t* v_cache, int max_pos, uint16_t* out, int ldo, void* ws,
                                  hipStream_t s, const uint32_t* frame_dev, int pos0,
                                  uint32_t* err);

// ---- frame helpers -------------------------------------------------------------
// audio_emb: HOST array of n_cb-1 device pointers (copied into the kernel arguments)
// Final draw of the last codebook from the head's per-block winners, then the
// frame embedding x' = bf16((E_tok[c0] + sum_j A_j[c_j]) * 8^-1/2), the code
// ring slot of this frame and the frame counter.
hipError_t launch_feedback(const uint16_t* tok_emb_audio, const uint16_t* const* audio_emb,
                           int32_t* codes, const Best* last_part, int last_nparts,
                           int32_t vocab_base, int n_slice, int code_vocab, int n_cb, int B,
                           int H, uint16_t* x_out, int32_t* ring, uint32_t* frame, int32_t end_id, uint32_t* stop,
                           hipStream_t s);
hipError_t launch_copy_bf16(const uint16_t* src, uint16_t* dst, size_t n, hipStream_t s);

// ---- persistent frame (persist.hip) -------------------------------------------
// A frame recorded as a table of phases (one GEMV each, then the frame end)
// and run as one cooperative launch.  Epoch of phase i of launch n: n *
// kPhaseStride + i + 1 (flags hold it, tagged words its low 16 bits).
constexpr uint32_t kPhaseStride = 512;
constexpr int kPersistFlags = 256;       // flag words (one per workgroup, at most 256)
struct PersistPlan;
struct PersistLaunch;
// what the frame end of a persistent launch needs about the tagged streams
struct FeedbackTags {
  int last_part_prod = -1;       // step that wrote the last draw's row-block winners
  const void* th = nullptr;      // tagged body residual stream
  int th_prod = -1;              // step that last wrote it
  uint16_t* h_out = nullptr;     // plain copy of it for the caller
  uint32_t* seq = nullptr;       // launch counter
  // (every frame path) the end token and the rows' stop words
  int32_t end_id = -1;
  uint32_t* stop = nullptr;
};
// An attention phase (persist_attn.h): q/k norm + RoPE with the cache write
// at the position, the chunks' partial softmax and their merge, for one body
// layer (position pos0 + *frame) or one depth layer (position pos).
struct AttnArgs {
  const uint32_t* qkv;     // the QKV GEMV's output words [B][ldqkv]
  const float* q_gamma;    // [128] per-head norm weights
  const float* k_gamma;
  const float* rope;       // [>= max_pos][64] (cos, sin)
  uint16_t* k_cache;       // bf16 [B][n_kv][max_pos][128]
  uint16_t* v_cache;
  uint32_t* out;           // output words [B][n_q * 128]
  uint64_t* rec;           // chunk records [B][n_kv][nchunks][G][2 + 128] (unused at nchunks 1)
  const uint32_t* frame;   // body: position pos0 + *frame; depth: nullptr (position pos)
  int ldqkv, n_q, n_kv, max_pos, pos0, pos, nchunks, ch, B;
  int pqkv;                // the phase that wrote qkv
  float eps, scale2;       // norm epsilon; log2(e) / sqrt(128) (set when recorded)
};
size_t persist_phase_bytes();
int persist_max_phases();
PersistPlan* persist_plan_new(int B);
void persist_plan_free(PersistPlan* pl);
int persist_plan_size(const PersistPlan* pl);
hipError_t persist_add_gemv(PersistPlan* pl, const GemvDesc& d);
hipError_t persist_add_feedback(PersistPlan* pl, const uint16_t* tok_emb_audio,
                                const uint16_t* const* audio_emb, int32_t* codes,
                                const Best* last_part, int last_nparts, int32_t vocab_base,
                                int n_slice, int code_vocab, int n_cb, int B, int H,
                                uint16_t* x_out, int32_t* ring, uint32_t* frame,
                                const FeedbackTags& ft);
hipError_t persist_add_attention(PersistPlan* pl, const AttnArgs& a);
// a guided draw phase (part: the winner records, written tagged; no ids or
// noise arrays): it waits for every workgroup to finish the step before it
hipError_t persist_add_cfg(PersistPlan* pl, const CfgDesc& d);
// phase clock: words of the buffer (3 per phase and workgroup), attach/detach
size_t persist_clock_words(const PersistLaunch& L);
void persist_set_clock(PersistLaunch& L, uint64_t* clk);
int persist_launch_dims(const PersistLaunch& L, int* nwg);   // phases; *nwg = workgroups
PersistLaunch* persist_launch_new();
void persist_launch_free(PersistLaunch* L);
// copy the table into device memory, start a new epoch (launch counter + 1),
// set the flags to its start and clear the error word (synchronises `s`)
hipError_t persist_upload(const PersistPlan* pl, void* table, uint32_t* flags, uint32_t* err,
                          uint32_t* seq, hipStream_t s, PersistLaunch* out);
hipError_t persist_launch(const PersistLaunch& L, hipStream_t s);
// the cooperative frame kernels (persist_bf16.hip, persist_i8row.hip,
// persist_fp8row.hip; with attention phases persist_*_attn.hip) (clock: the
// instantiation that writes the phase clock; every row count runs on 16-row
// tiles)
const void* persist_kernel_bf16(bool clock, bool attn);
const void* persist_kernel_i8row(bool clock, bool attn);
const void* persist_kernel_fp8row(bool clock, bool attn);
const void* persist_kernel_bf16_attn(bool clock);
const void* persist_kernel_i8row_attn(bool clock);
const void* persist_kernel_fp8row_attn(bool clock);
hipError_t launch_fill_u32(uint32_t* dst, uint32_t v, size_t n, hipStream_t s);
// a plain streaming read of `bytes` (< 2 GiB) at buf by `workgroups` workgroups
// (stream.hip); sink: workgroups words
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                              int nontemporal, hipStream_t s);

}  // namespace m3
