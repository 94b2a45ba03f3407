// capi.cpp -- the C ABI of libm3: host-side validation, then launches.
//
// Every entry point checks its arguments before touching the GPU and returns
// a negative m3_status without enqueuing anything when they fall outside the
// supported set (TensorFold PR #987, "Kernel contract": unsupported edges are
// refused; DiffSynth-Studio's MiniMax-Music3 parameters: invalid input raises
// instead of proceeding).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "m3_internal.h"

#include <vector>

using namespace m3;

namespace {

constexpr size_t kLdsMax = 160 * 1024;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int k_ok(int fmt, int K) {
  if (K < 8) return 0;
  switch (fmt) {
    case M3_BF16: return K % 8 == 0;
    case M3_I8ROW:
    case M3_FP8ROW: return K % 16 == 0;
    case M3_I8G128: return K % 128 == 0;
    default: return 0;
  }
}

bool fmt_ok(int fmt) {
  return fmt == M3_BF16 || fmt == M3_I8ROW || fmt == M3_I8G128 || fmt == M3_FP8ROW;
}

// formats of a whole-row-scale matrix (body, lm_head)
bool row_fmt(int fmt) { return fmt == M3_BF16 || fmt == M3_I8ROW || fmt == M3_FP8ROW; }

int hip_status(hipError_t e) { return e == hipSuccess ? M3_OK : M3_ERR_HIP; }

// [a0, a1) and [b0, b1) overlap?
bool overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

int validate_gemv(int fmt, const void* w, int N, int K, const uint16_t* x, int B, int ldx,
                  const float* gamma, float eps, int stub_group, int stub_voff, void* y,
                  int ldy, int out_dtype, int epi, const uint16_t* res, int ldr) {
  if (!w || !x || !y) return M3_ERR_NULL;
  if (!fmt_ok(fmt)) return M3_ERR_FORMAT;
  if (out_dtype != M3_OUT_BF16 && out_dtype != M3_OUT_F32) return M3_ERR_FORMAT;
  if (epi != M3_EPI_NONE && epi != M3_EPI_SWIGLU && epi != M3_EPI_RESIDUAL) return M3_ERR_FORMAT;
  if (epi != M3_EPI_NONE && out_dtype != M3_OUT_BF16) return M3_ERR_FORMAT;
  if (N < 1 || !k_ok(fmt, K) || B < 1 || B > M3_MAX_B) return M3_ERR_SHAPE;
  if (epi == M3_EPI_SWIGLU && (N % 2) != 0) return M3_ERR_SHAPE;
  if (epi == M3_EPI_RESIDUAL && !res) return M3_ERR_NULL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return M3_ERR_SHAPE;
  // operand columns read from x
  long need_ldx = K;
  if (stub_group < 0) return M3_ERR_SHAPE;
  if (stub_group > 0) {
    if (K % 128 != 0 || (K / 128) % stub_group != 0 || stub_voff < 0 || stub_voff % 8 != 0)
      return M3_ERR_SHAPE;
    need_ldx = (long)stub_voff + (long)(K / 128 / stub_group) * 128;
  }
  if (ldx < need_ldx) return M3_ERR_SHAPE;
  const int ncols = epi == M3_EPI_SWIGLU ? N / 2 : N;
  if (ldy < ncols) return M3_ERR_SHAPE;
  if (epi == M3_EPI_RESIDUAL && ldr < N) return M3_ERR_SHAPE;
  if (ldx % 8 != 0 || ldy % 8 != 0 || (epi == M3_EPI_RESIDUAL && ldr % 8 != 0)) return M3_ERR_ALIGN;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 16)) return M3_ERR_ALIGN;
  if (gamma && !aligned(gamma, 16)) return M3_ERR_ALIGN;
  if (res && !aligned(res, 16)) return M3_ERR_ALIGN;
  if (gamma && (long)B * k_pad(fmt, K) > kMaxNormElems) return M3_ERR_SHAPE;
  if (gemv_smem_bytes(fmt, K, B, gamma != nullptr) > kLdsMax) return M3_ERR_SHAPE;
  // x is read by every workgroup while outputs are written: no overlap
  const size_t esz = out_dtype == M3_OUT_F32 ? 4 : 2;
  const size_t xbytes = ((size_t)(B - 1) * ldx + need_ldx) * 2;
  const size_t ybytes = ((size_t)(B - 1) * ldy + ncols) * esz;
  if (overlap(x, xbytes, y, ybytes)) return M3_ERR_ALIAS;
  if (epi == M3_EPI_RESIDUAL && res != y) {
    const size_t rbytes = ((size_t)(B - 1) * ldr + N) * 2;
    if (overlap(res, rbytes, y, ybytes)) return M3_ERR_ALIAS;
  }
  if (epi == M3_EPI_RESIDUAL && res == y && ldr != ldy) return M3_ERR_ALIAS;
  return M3_OK;
}

int gemv_entry(int fmt, const void* w, int N, int K, const uint16_t* x, int B, int ldx,
               const float* gamma, float eps, int stub_group, int stub_voff, void* y, int ldy,
               int out_dtype, int epi, const uint16_t* res, int ldr, void* stream) {
  const int st = validate_gemv(fmt, w, N, K, x, B, ldx, gamma, eps, stub_group, stub_voff, y,
                               ldy, out_dtype, epi, res, ldr);
  if (st != M3_OK) return st;
  GemvDesc d{fmt, w, N, K, x, ldx, B, gamma, eps, stub_group, stub_voff, y, ldy,
             out_dtype == M3_OUT_F32, epi, res, ldr};
  return hip_status(launch_gemv(d, static_cast<hipStream_t>(stream)));
}

// ---- frame -------------------------------------------------------------------
struct Dims {
  int H, nq, nkv, nqkv, F, D, dq, dqkv, Fd, V0, CV, ncb;
  int e;       // 1: the lm_head's row 0 is the end token
  int VL, ldl; // lm_head rows (V0 + e) and the logits' row stride
};

Dims dims_of(const m3_config& c) {
  Dims d;
  d.H = c.hidden;
  d.nq = c.n_heads * c.head_dim;
  d.nkv = c.n_kv_heads * c.head_dim;
  d.nqkv = d.nq + 2 * d.nkv;
  d.F = c.ffn;
  d.D = c.d_hidden;
  d.dq = c.d_heads * c.d_head_dim;
  d.dqkv = 3 * d.dq;
  d.Fd = c.d_ffn;
  d.V0 = c.n_slice;
  d.CV = c.code_vocab;
  d.ncb = c.n_codebooks;
  d.e = c.end_id >= 0 ? 1 : 0;
  d.VL = d.V0 + d.e;
  d.ldl = (d.VL + 7) / 8 * 8;
  return d;
}

uint64_t mat_bytes(int fmt, uint64_t N, uint64_t K) {
  if (fmt == M3_BF16) return 2 * N * K;
  if (fmt == M3_I8ROW || fmt == M3_FP8ROW) return N * K + 4 * N;
  return N * K + 4 * N * (K / 128);
}

int validate_config(const m3_config* c, int B) {
  if (!c) return M3_ERR_NULL;
  if (!fmt_ok(c->fmt_body) || !fmt_ok(c->fmt_depth)) return M3_ERR_FORMAT;
  if (!row_fmt(c->fmt_lm)) return M3_ERR_FORMAT;
  if (B < 1 || B > M3_MAX_B_FRAME) return M3_ERR_SHAPE;
  if (c->n_layers < 1 || c->d_layers < 1) return M3_ERR_SHAPE;
  // the reference's draw: rows in (conditional, unconditional) pairs
  if (c->top_k < 0) return M3_ERR_SHAPE;
  if (c->top_k > 0 && (B % 2 != 0 || !std::isfinite(c->cfg_scale) || c->n_slice > M3_MAX_V_CFG ||
                       c->code_vocab > M3_MAX_V_CFG))
    return M3_ERR_SHAPE;
  if (c->head_dim != 128 || c->d_head_dim != 128) return M3_ERR_SHAPE;
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads) return M3_ERR_SHAPE;
  if (c->d_heads < 1) return M3_ERR_SHAPE;
  if (c->n_codebooks < 2 || c->n_codebooks > 8) return M3_ERR_SHAPE;
  if (c->n_slice < 1 || c->code_vocab < 1 || c->vocab_base < 0) return M3_ERR_SHAPE;
  // the end token sorts before the codes (row 0 of the lm_head)
  if (c->end_id >= c->vocab_base || (c->end_id >= 0 && c->top_k > 0 && c->n_slice + 1 > M3_MAX_V_CFG))
    return M3_ERR_SHAPE;
  if (!(c->temperature > 0.0f) || !std::isfinite(c->temperature)) return M3_ERR_SHAPE;
  if (!(c->eps >= 0.0f) || !std::isfinite(c->eps)) return M3_ERR_SHAPE;
  const Dims d = dims_of(*c);
  const int fb = c->fmt_body, fd = c->fmt_depth;
  // every K a GEMV of the frame contracts over
  if (!k_ok(fb, d.H) || !k_ok(fb, d.nq) || !k_ok(fb, d.F)) return M3_ERR_SHAPE;
  if (!k_ok(c->fmt_lm, d.H) || !k_ok(fd, d.H)) return M3_ERR_SHAPE;
  if (!k_ok(fd, d.D) || !k_ok(fd, d.dq) || !k_ok(fd, d.Fd)) return M3_ERR_SHAPE;
  // leading dimensions are multiples of 8 elements
  if (d.H % 8 || d.nqkv % 8 || d.F % 8 || d.D % 8 || d.dqkv % 8 || d.Fd % 8 || d.V0 % 8 ||
      d.CV % 8)
    return M3_ERR_SHAPE;
  // norm-fused GEMVs must fit LDS
  if ((long)B * k_pad(fb, d.H) > kMaxNormElems || (long)B * k_pad(fd, d.D) > kMaxNormElems ||
      (long)B * k_pad(c->fmt_lm, d.H) > kMaxNormElems || (long)B * k_pad(fd, d.H) > kMaxNormElems)
    return M3_ERR_SHAPE;
  if (gemv_smem_bytes(fb, d.H, B, true) > kLdsMax || gemv_smem_bytes(c->fmt_lm, d.H, B, true) > kLdsMax ||
      gemv_smem_bytes(fd, d.H, B, true) > kLdsMax || gemv_smem_bytes(fd, d.D, B, true) > kLdsMax)
    return M3_ERR_SHAPE;
  if (c->n_layers > 1000 || c->d_layers > 1000) return M3_ERR_SHAPE;
  // decode attention over the frame state's caches
  if (c->attention != 0 && c->attention != 1) return M3_ERR_SHAPE;
  if (c->attention) {
    if (c->max_pos < 1 || c->max_pos > M3_MAX_POS || c->pos0 < 0 || c->pos0 >= c->max_pos)
      return M3_ERR_SHAPE;
    const int g = c->n_heads / c->n_kv_heads;
    if ((g != 1 && g != 2 && g != 4 && g != 8) || c->n_heads > M3_MAX_HEADS ||
        c->d_heads > M3_MAX_HEADS)
      return M3_ERR_SHAPE;
  }
  return M3_OK;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// phases of one frame: 4 GEMVs per body layer, lm_head, depth input, per depth
// step 4 GEMVs per layer and the head, then the frame end; with decode
// attention one attention phase per body layer and per depth layer run; with
// the guided draw one draw phase after the lm_head and after each head
int frame_phases(const m3_config& c) {
  const int per_layer = c.attention ? 5 : 4;
  const int draws = c.top_k > 0 ? c.n_codebooks : 0;     // guided draws: semantic + depth heads
  return per_layer * c.n_layers + 2 + (c.n_codebooks - 1) * (per_layer * c.d_layers + 1) + draws + 1;
}

// the body's decode attention at T = max_pos: positions per chunk and chunks
// (the chunk records of a persistent frame are sized for them)
int body_attn_chunk(const m3_config& c, int B) { return attn_chunk_size(B, c.n_kv_heads, c.max_pos); }
int body_attn_chunks(const m3_config& c, int B) {
  const int ch = body_attn_chunk(c, B);
  return (c.max_pos + ch - 1) / ch;
}

m3_frame_layout layout_of(const m3_config& c, int B) {
  const Dims d = dims_of(c);
  m3_frame_layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  // Per-stage slots: every GEMV output of every body layer and of every
  // depth layer of every codebook step has a slot of its own (nothing is
  // overwritten within a frame), plus per depth step its input and each
  // head's logits.
  const size_t nL = (size_t)c.n_layers;
  const size_t nS = (size_t)(d.ncb - 1);               // depth steps
  const size_t nDL = nS * c.d_layers;                  // depth layers run per frame
  const size_t nHD = nS * (c.d_layers + 1);            // depth residual slots
  L.x = take((size_t)B * d.H * 2);
  L.h = take(nL * B * d.H * 2);
  L.qkv = take(nL * B * d.nqkv * 2);
  L.mlp = take(nL * B * d.F * 2);
  L.logits = take((size_t)B * d.ldl * 4);
  L.u = take((size_t)B * d.D * 2);
  L.hd = take(nHD * B * d.D * 2);
  L.dqkv = take(nDL * B * d.dqkv * 2);
  L.dmlp = take(nDL * B * d.Fd * 2);
  L.dlogits = take(nS * B * d.CV * 4);
  L.ring = take((size_t)16 * B * 8 * 4);
  L.frame = take(4);
  L.part_sem = take((size_t)B * n_blocks(d.VL) * sizeof(Best));
  // one set of row-block winners per depth step (each is read by the next
  // step's gather and the frame end; none is written twice in a frame)
  L.part_dep = take((size_t)(d.ncb - 1) * B * n_blocks(d.CV) * sizeof(Best));
  L.flags = take((size_t)kPersistFlags * 4);
  L.err = take(4);
  L.seq = take(4);
  L.phases = take((size_t)frame_phases(c) * persist_phase_bytes());
  L.th = take(nL * B * d.H * 4);
  L.tqkv = take(nL * B * d.nqkv * 4);
  L.tmlp = take(nL * B * d.F * 4);
  L.tu = take((size_t)B * d.D * 4);
  L.thd = take(nHD * B * d.D * 4);
  L.tdqkv = take(nDL * B * d.dqkv * 4);
  L.tdmlp = take(nDL * B * d.Fd * 4);
  L.th2 = take(nL * B * d.H * 4);
  L.thd2 = take(nDL * B * d.D * 4);
  L.ho = take(nL * B * d.H * 2);
  L.hdo = take(nDL * B * d.D * 2);
  const bool at = c.attention != 0;
  const int rope_pos = at ? std::max(c.max_pos, 8) : 0;
  L.rope = take((size_t)rope_pos * 64 * 2 * 4);
  L.aq = take(at ? (size_t)B * std::max(d.nq, d.dq) * 2 : 0);
  L.ao = take(at ? nL * B * d.nq * 2 : 0);
  L.dao = take(at ? nDL * B * d.dq * 2 : 0);
  const size_t kv = at ? (size_t)c.n_layers * B * c.n_kv_heads * c.max_pos * 128 * 2 : 0;
  L.kcache = take(kv);
  L.vcache = take(kv);
  const size_t dkv = at ? (size_t)c.d_layers * B * c.d_heads * 8 * 128 * 2 : 0;
  L.dkcache = take(dkv);
  L.dvcache = take(dkv);
  L.attn_ws = take(at ? attn_workspace_bytes(B, c.n_heads, c.n_kv_heads, c.max_pos) : 0);
  // the persistent frame's attention outputs (u32 words) and, per body layer,
  // its chunk records (tagged 64-bit words)
  L.tao = take(at ? nL * B * d.nq * 4 : 0);
  L.tdao = take(at ? nDL * B * d.dq * 4 : 0);
  const int nch = at ? body_attn_chunks(c, B) : 0;
  L.trec = take(at && nch > 1 ? nL * B * c.n_heads * nch * (2 + 128) * 8 : 0);
  L.stop = take((size_t)B * 4);
  // the eager and graph frames' GEMVs split along K (gemv.hip): the down
  // projections, whose outputs have max(H, D) rows at most
  const int kblocks = n_blocks(std::max(d.H, d.D));
  L.kpart = take(gemv_split_part_bytes(kblocks));
  L.kcnt = take(gemv_split_counters(kblocks) * 4);
  L.total = off;
  return L;
}

int validate_model(const m3_model* m) {
  if (!m || !m->layers || !m->final_norm || !m->lm_head || !m->p_in || !m->emb1 ||
      !m->d_layers_w || !m->d_final_norm || !m->heads || !m->tok_emb_audio || !m->audio_emb)
    return M3_ERR_NULL;
  if (m->cfg.n_codebooks > 2 && !m->emb) return M3_ERR_NULL;
  for (int l = 0; l < m->cfg.n_layers; ++l) {
    const m3_layer_weights& L = m->layers[l];
    if (!L.qkv || !L.o || !L.gate_up || !L.down || !L.attn_norm || !L.ffn_norm) return M3_ERR_NULL;
  }
  for (int l = 0; l < m->cfg.d_layers; ++l) {
    const m3_layer_weights& L = m->d_layers_w[l];
    if (!L.qkv || !L.o || !L.gate_up || !L.down || !L.attn_norm || !L.ffn_norm) return M3_ERR_NULL;
  }
  if (m->cfg.attention) {
    for (int l = 0; l < m->cfg.n_layers; ++l)
      if (!m->layers[l].q_norm || !m->layers[l].k_norm) return M3_ERR_NULL;
    for (int l = 0; l < m->cfg.d_layers; ++l)
      if (!m->d_layers_w[l].q_norm || !m->d_layers_w[l].k_norm) return M3_ERR_NULL;
  }
  for (int j = 0; j < m->cfg.n_codebooks - 1; ++j)
    if (!m->heads[j] || !m->audio_emb[j]) return M3_ERR_NULL;
  for (int j = 0; j < m->cfg.n_codebooks - 2; ++j)
    if (!m->emb[j]) return M3_ERR_NULL;
  return M3_OK;
}

#define M3_TRY(expr)                         \
  do {                                       \
    const hipError_t e_ = (expr);            \
    if (e_ != hipSuccess) return M3_ERR_HIP; \
  } while (0)

// Where the frame's steps go: launched one kernel each on a stream, or recorded
// as the phases of one persistent launch.
// one attention step of the frame: q/k norm + RoPE with the cache write, then
// attention over the cache (frame_dev set: the position comes from the frame
// counter; otherwise pos)
struct AttnStep {
  const uint16_t* qkv;
  int ldqkv, n_q, n_kv;
  const float *q_gamma, *k_gamma;
  float eps;
  const float* rope;
  int pos;
  uint16_t *q, *k_cache, *v_cache, *out;
  int max_pos;
  const uint32_t* frame_dev;
  int pos0;
  uint32_t* err;
  void* ws;
  // a persistent frame's step: the phase that wrote qkv (tagged words), the
  // output words, the chunk records (body) and this layer's index
  int pqkv = -1;
  uint32_t* tout = nullptr;
  uint64_t* rec = nullptr;
  int B = 0;
};

struct FrameSink {
  virtual hipError_t gemv(const GemvDesc& d) = 0;
  virtual hipError_t cfg_draw(const CfgDesc& d) = 0;
  virtual hipError_t attention(const AttnStep& a, int B) = 0;
  virtual hipError_t feedback(const uint16_t* tok, const uint16_t* const* aemb, int32_t* codes,
                              const Best* last_part, int last_nparts, int32_t vocab_base,
                              int n_slice, int code_vocab, int n_cb, int B, int H, uint16_t* x,
                              int32_t* ring, uint32_t* frame, const FeedbackTags& ft) = 0;
};

struct LaunchSink final : FrameSink {
  hipStream_t s;
  explicit LaunchSink(hipStream_t st) : s(st) {}
  hipError_t gemv(const GemvDesc& d) override { return launch_gemv(d, s); }
  hipError_t cfg_draw(const CfgDesc& d) override { return launch_cfg_draw(d, s); }
  hipError_t attention(const AttnStep& a, int B) override {
    return launch_attention_fused(a.qkv, B, a.ldqkv, a.n_q, a.n_kv, a.q_gamma, a.k_gamma, a.eps,
                                  a.rope, a.pos, a.k_cache, a.v_cache, a.max_pos, a.out,
                                  a.n_q * 128, a.ws, s, a.frame_dev, a.pos0, a.err);
  }
  hipError_t feedback(const uint16_t* tok, const uint16_t* const* aemb, int32_t* codes,
                      const Best* last_part, int last_nparts, int32_t vocab_base, int n_slice,
                      int code_vocab, int n_cb, int B, int H, uint16_t* x, int32_t* ring,
                      uint32_t* frame, const FeedbackTags& ft) override {
    return launch_feedback(tok, aemb, codes, last_part, last_nparts, vocab_base, n_slice,
                           code_vocab, n_cb, B, H, x, ring, frame, ft.end_id, ft.stop, s);
  }
};

// chunks of a frame-position (body) attention step's records
int body_attn_chunks_of(const AttnStep& s, int B) {
  const int ch = attn_chunk_size(B, s.n_kv, s.max_pos);
  return (s.max_pos + ch - 1) / ch;
}

// a persistent frame's attention phase, chunked as the decode attention
// launches chunk (T = max_pos for a body layer, pos + 1 for a depth layer)
AttnArgs attn_args(const AttnStep& s, int B) {
  AttnArgs a{};
  a.qkv = reinterpret_cast<const uint32_t*>(s.qkv);
  a.q_gamma = s.q_gamma;
  a.k_gamma = s.k_gamma;
  a.rope = s.rope;
  a.k_cache = s.k_cache;
  a.v_cache = s.v_cache;
  a.out = s.tout;
  a.rec = s.rec;
  a.frame = s.frame_dev;
  a.ldqkv = s.ldqkv;
  a.n_q = s.n_q;
  a.n_kv = s.n_kv;
  a.max_pos = s.max_pos;
  a.pos0 = s.pos0;
  a.pos = s.pos;
  const int Tg = s.frame_dev ? s.max_pos : s.pos + 1;
  a.ch = attn_chunk_size(B, s.n_kv, Tg);
  a.nchunks = (Tg + a.ch - 1) / a.ch;
  a.B = B;
  a.pqkv = s.pqkv;
  a.eps = s.eps;
  return a;
}

struct PlanSink final : FrameSink {
  PersistPlan* pl;
  explicit PlanSink(PersistPlan* p) : pl(p) {}
  hipError_t gemv(const GemvDesc& d) override { return persist_add_gemv(pl, d); }
  hipError_t cfg_draw(const CfgDesc& d) override { return persist_add_cfg(pl, d); }
  hipError_t attention(const AttnStep& s, int B) override { return persist_add_attention(pl, attn_args(s, B)); }
  hipError_t feedback(const uint16_t* tok, const uint16_t* const* aemb, int32_t* codes,
                      const Best* last_part, int last_nparts, int32_t vocab_base, int n_slice,
                      int code_vocab, int n_cb, int B, int H, uint16_t* x, int32_t* ring,
                      uint32_t* frame, const FeedbackTags& ft) override {
    return persist_add_feedback(pl, tok, aemb, codes, last_part, last_nparts, vocab_base, n_slice,
                                code_vocab, n_cb, B, H, x, ring, frame, ft);
  }
};

// The frame's steps in order.  tagged: the steps of a persistent launch,
// whose intermediate streams are the tagged buffers of the state (32-bit
// words carrying the producing phase, see gemv_impl.h) and whose GEMVs are
// told which phase produced each of their inputs.
int build_frame(const m3_model* m, uint8_t* S, int B, int32_t* codes, FrameSink& sink,
                bool tagged = false) {
  const m3_config& c = m->cfg;
  const Dims d = dims_of(c);
  const m3_frame_layout L = layout_of(c, B);
  // Every stream has one slot per layer (body) or per depth step and layer
  // (depth decoder): plain bf16 in the eager/graph frames, tagged 32-bit
  // words in a persistent launch.  Nothing is written twice within a frame,
  // so no consumer can see a buffer overwritten under it.
  const size_t esz = tagged ? 4 : 2;
  auto slot = [&](size_t plain, size_t tag, size_t i, size_t cols) {
    return reinterpret_cast<uint16_t*>(S + (tagged ? tag : plain) + i * B * cols * esz);
  };
  uint16_t* x = reinterpret_cast<uint16_t*>(S + L.x);
  // body layer l: QKV output, the stream after O (h_o), SwiGLU output, the
  // stream after down (h); the body output is the last layer's h
  auto h_slot = [&](int l) { return slot(L.h, L.th, l, d.H); };
  auto qkv_slot = [&](int l) { return slot(L.qkv, L.tqkv, l, d.nqkv); };
  auto ho_slot = [&](int l) { return slot(L.ho, L.th2, l, d.H); };
  auto mlp_slot = [&](int l) { return slot(L.mlp, L.tmlp, l, d.F); };
  uint16_t* h_out = h_slot(c.n_layers - 1);
  uint16_t* h_plain_out = reinterpret_cast<uint16_t*>(S + L.h + (size_t)(c.n_layers - 1) * B * d.H * 2);
  float* logits = reinterpret_cast<float*>(S + L.logits);
  uint16_t* u = slot(L.u, L.tu, 0, d.D);
  // depth step j (1-based): residual slot s (0 = the step input, l + 1 =
  // after depth layer l) and the per-layer streams of layer l
  auto hd_slot = [&](int j, int s) {
    return slot(L.hd, L.thd, (size_t)(j - 1) * (c.d_layers + 1) + s, d.D);
  };
  auto dl_index = [&](int j, int l) { return (size_t)(j - 1) * c.d_layers + l; };
  auto dqkv_slot = [&](int j, int l) { return slot(L.dqkv, L.tdqkv, dl_index(j, l), d.dqkv); };
  auto hdo_slot = [&](int j, int l) { return slot(L.hdo, L.thd2, dl_index(j, l), d.D); };
  auto dmlp_slot = [&](int j, int l) { return slot(L.dmlp, L.tdmlp, dl_index(j, l), d.Fd); };
  auto dlogits_of = [&](int j) {
    return reinterpret_cast<float*>(S + L.dlogits) + (size_t)(j - 1) * B * d.CV;
  };
  int32_t* ring = reinterpret_cast<int32_t*>(S + L.ring);
  uint32_t* frame = reinterpret_cast<uint32_t*>(S + L.frame);
  Best* part_sem = reinterpret_cast<Best*>(S + L.part_sem);
  // depth step j's (1-based) row-block winners
  auto part_dep = [&](int j) {
    return reinterpret_cast<Best*>(S + L.part_dep) + (size_t)(j - 1) * B * n_blocks(d.CV);
  };
  const float eps = c.eps;
  // index of the next step, and the step that last wrote each stream (-1:
  // none in this frame; the frame input is a plain buffer)
  int ph = 0;
  int p_h = -1, p_qkv = -1, p_mlp = -1, p_u = -1, p_hd = -1, p_dqkv = -1, p_dmlp = -1;
  (void)p_mlp;
  (void)p_dmlp;
  int p_sem = -1, p_dep = -1;
  struct Prod {
    int x = -1, res = -1, u = -1, part = -1;
  };
  // Scheduling of a persistent launch (values unchanged): with the attention
  // stub, O reads only the V rows of QKV, so QKV takes its V row blocks first
  // (rot) and O starts while the workgroups with a second QKV block finish
  // it; the depth decoder's O (fewer blocks than workgroups) goes to the
  // workgroups that had one QKV block (follow).
  struct Sched {
    int rot = 0, follow = 0;
  };
  auto gemv = [&](int fmt, const void* w, int N, int K, const uint16_t* xin, int ldx,
                  const float* gamma, int sg, int sv, void* y, int ldy, int f32, int epi,
                  const uint16_t* res, int ldr, Prod pr, const SampleEpi* smp = nullptr,
                  const GatherPro* gat = nullptr, Sched sc = Sched{}) {
    GemvDesc g{fmt, w, N, K, xin, ldx, B, gamma, eps, sg, sv, y, ldy, f32, epi, res, ldr, smp, gat};
    if (tagged) {
      g.px = pr.x;
      g.pres = pr.res;
      g.pu = pr.u;
      g.ppart = pr.part;
      g.ytag = 1;
      g.rot = sc.rot;
      g.follow = sc.follow;
    } else {
      g.kpart = reinterpret_cast<float*>(S + L.kpart);
      g.kcnt = reinterpret_cast<uint32_t*>(S + L.kcnt);
      g.kpart_blocks = n_blocks(std::max(d.H, d.D));
    }
    const hipError_t e = sink.gemv(g);
    ++ph;
    return e;
  };
  // ---- attention (c.attention == 1): caches and buffers of the state ----
  const bool attn = c.attention != 0;
  const float* rope = reinterpret_cast<const float*>(S + L.rope);
  uint16_t* aq = reinterpret_cast<uint16_t*>(S + L.aq);
  uint32_t* err = reinterpret_cast<uint32_t*>(S + L.err);
  // attention outputs: one slot per body layer (ao) and per depth layer run (dao)
  auto ao_slot = [&](int l) { return reinterpret_cast<uint16_t*>(S + L.ao + (size_t)l * B * d.nq * 2); };
  auto dao_slot = [&](int j, int l) {
    return reinterpret_cast<uint16_t*>(S + L.dao + dl_index(j, l) * B * d.dq * 2);
  };
  // (a persistent frame: the output words tao / tdao, the chunk records trec)
  auto tao_slot = [&](int l) { return reinterpret_cast<uint32_t*>(S + L.tao) + (size_t)l * B * d.nq; };
  auto tdao_slot = [&](int j, int l) {
    return reinterpret_cast<uint32_t*>(S + L.tdao) + dl_index(j, l) * B * d.dq;
  };
  auto rec_slot = [&](int l) {
    const size_t per = (size_t)B * c.n_heads * body_attn_chunks(c, B) * (2 + 128);
    return L.trec ? reinterpret_cast<uint64_t*>(S + L.trec) + (size_t)l * per : nullptr;
  };
  auto attention = [&](const uint16_t* qkv_in, int ldq_in, int n_q, int n_kv,
                       const m3_layer_weights& W, uint16_t* kc, uint16_t* vc, int max_pos,
                       int pos, bool from_frame, uint16_t* ao, int pq, uint32_t* tout,
                       uint64_t* rec) {
    AttnStep a{qkv_in, ldq_in, n_q, n_kv, W.q_norm, W.k_norm, eps, rope, pos, aq, kc, vc, ao,
               max_pos, from_frame ? frame : nullptr, from_frame ? c.pos0 : 0, err,
               S + L.attn_ws};
    if (tagged) {
      a.pqkv = pq;
      a.tout = tout;
      a.rec = rec;
    }
    a.B = B;
    ++ph;
    return sink.attention(a, B);
  };
  // ---- body ----
  const int group = c.n_heads / c.n_kv_heads;
  for (int l = 0; l < c.n_layers; ++l) {
    const m3_layer_weights& W = m->layers[l];
    const uint16_t* xin = l == 0 ? x : h_slot(l - 1);
    uint16_t* h = h_slot(l);
    uint16_t* qkv = qkv_slot(l);
    uint16_t* h_o = ho_slot(l);
    uint16_t* mlp = mlp_slot(l);
    uint16_t* ao = attn ? ao_slot(l) : nullptr;
    const int p_xin = l == 0 ? -1 : p_h;
    Prod a;
    a.x = p_xin;
    p_qkv = ph;
    Sched qs;
    if (!attn) qs.rot = (d.nq + d.nkv) / 16;      // the first V row block
    M3_TRY(gemv(c.fmt_body, W.qkv, d.nqkv, d.H, xin, d.H, W.attn_norm, 0, 0, qkv, d.nqkv, 0,
                M3_EPI_NONE, nullptr, 0, a, nullptr, nullptr, qs));
    Prod o;
    o.x = p_qkv;
    o.res = p_xin;
    int p_ho;
    if (attn) {
      const size_t lay = (size_t)B * c.n_kv_heads * c.max_pos * 128 * 2;
      o.x = ph;                                    // O reads the attention's output
      M3_TRY(attention(qkv, d.nqkv, c.n_heads, c.n_kv_heads, W,
                       reinterpret_cast<uint16_t*>(S + L.kcache + l * lay),
                       reinterpret_cast<uint16_t*>(S + L.vcache + l * lay), c.max_pos, 0, true,
                       ao, p_qkv, tao_slot(l), rec_slot(l)));
      p_ho = ph;
      M3_TRY(gemv(c.fmt_body, W.o, d.H, d.nq, tagged ? reinterpret_cast<uint16_t*>(tao_slot(l)) : ao,
                  d.nq, nullptr, 0, 0, h_o, d.H, 0, M3_EPI_RESIDUAL, xin, d.H, o));
    } else {
      p_ho = ph;
      M3_TRY(gemv(c.fmt_body, W.o, d.H, d.nq, qkv, d.nqkv, nullptr, group, d.nq + d.nkv, h_o, d.H,
                  0, M3_EPI_RESIDUAL, xin, d.H, o));
    }
    Prod gu;
    gu.x = p_ho;
    p_mlp = ph;
    M3_TRY(gemv(c.fmt_body, W.gate_up, 2 * d.F, d.H, h_o, d.H, W.ffn_norm, 0, 0, mlp, d.F, 0,
                M3_EPI_SWIGLU, nullptr, 0, gu));
    Prod dn;
    dn.x = p_mlp;
    dn.res = p_ho;
    p_h = ph;
    M3_TRY(gemv(c.fmt_body, W.down, d.H, d.F, mlp, d.F, nullptr, 0, 0, h, d.H, 0,
                M3_EPI_RESIDUAL, h_o, d.H, dn));
  }
  // The reference's draw (top_k > 0): guidance over (conditional,
  // unconditional) row pairs, top-k, Gumbel-argmax; one draw per song, left
  // as a one-entry winner record per row for the same consumers.
  const bool guided = c.top_k > 0;
  auto guided_draw = [&](const float* lg, int V, int ldl, uint32_t draw, int32_t base,
                         int32_t end_id, Best* part) {
    CfgDesc g{};
    g.logits = lg;
    g.S = B / 2;
    g.V = V;
    g.ldl = ldl;
    g.end_id = end_id;
    g.scale = c.cfg_scale;
    g.top_k = c.top_k;
    g.seed = c.seed;
    g.frame_dev = frame;
    g.draw = draw;
    g.temperature = c.temperature;
    g.index_base = base;
    g.part = part;
    g.out_stride = 1;
    g.vec4 = ldl % 4 == 0;
    ++ph;
    return sink.cfg_draw(g);
  };
  // ---- sliced lm_head; its epilogue adds the Gumbel noise of draw 0 and
  // leaves each row block's winner; the draw completes in the next consumer
  // (with the end token: column 0 is it, column 1 + i code i)
  const int32_t end_id = d.e ? c.end_id : -1;
  const int32_t lm_base = c.vocab_base - d.e;     // absolute id of column n >= e is lm_base + n
  SampleEpi sem{c.seed, frame, 0u, c.temperature, lm_base, c.vocab_base,
                c.vocab_base + c.n_slice, part_sem, end_id};
  Prod lm;
  lm.x = p_h;
  p_sem = ph;
  M3_TRY(gemv(c.fmt_lm, m->lm_head, d.VL, d.H, h_out, d.H, m->final_norm, 0, 0, logits, d.ldl, 1,
              M3_EPI_NONE, nullptr, 0, lm, guided ? nullptr : &sem));
  if (guided) {
    p_sem = ph;                     // the draw writes the winner records
    M3_TRY(guided_draw(logits, d.VL, d.ldl, 0u, lm_base, end_id, part_sem));
  }
  // ---- depth decoder ----
  Prod pin;
  pin.x = p_h;
  p_u = ph;
  M3_TRY(gemv(c.fmt_depth, m->p_in, d.D, d.H, h_out, d.H, m->final_norm, 0, 0, u, d.D, 0,
              M3_EPI_NONE, nullptr, 0, pin));
  for (int j = 1; j < d.ncb; ++j) {
    float* dlogits = dlogits_of(j);
    // step j's input: bf16(u + Emb_j[previous code]); the previous draw is
    // finished from its row-block winners in the prologue of the first GEMV
    GatherPro gp;
    gp.u = u;
    gp.emb = j == 1 ? m->emb1 : m->emb[j - 2];
    gp.part = j == 1 ? part_sem : part_dep(j - 1);
    gp.nparts = guided ? 1 : (j == 1 ? n_blocks(d.VL) : n_blocks(d.CV));
    gp.index_base = j == 1 ? lm_base : 0;
    gp.end_id = j == 1 ? end_id : -1;
    gp.code_base = j == 1 ? c.vocab_base : 0;
    gp.n_codes = j == 1 ? c.n_slice : c.code_vocab;
    gp.codes = codes;
    gp.code_col = j - 1;
    gp.out = hd_slot(j, 0);
    const int p_prev_draw = j == 1 ? p_sem : p_dep;
    for (int l = 0; l < c.d_layers; ++l) {
      const m3_layer_weights& W = m->d_layers_w[l];
      uint16_t* hd = hd_slot(j, l);          // this layer's input
      uint16_t* hd_next = hd_slot(j, l + 1);  // and its output
      uint16_t* dqkv = dqkv_slot(j, l);
      uint16_t* hd_o = hdo_slot(j, l);
      uint16_t* dmlp = dmlp_slot(j, l);
      uint16_t* ao = attn ? dao_slot(j, l) : nullptr;
      Prod q;
      if (l == 0) {
        q.u = p_u;
        q.part = p_prev_draw;
        p_hd = ph;              // the gather writes the step's residual stream
      } else {
        q.x = p_hd;
      }
      p_dqkv = ph;
      Sched qs;
      if (!attn) qs.rot = 2 * d.dq / 16;           // the first V row block
      M3_TRY(gemv(c.fmt_depth, W.qkv, d.dqkv, d.D, hd, d.D, W.attn_norm, 0, 0, dqkv, d.dqkv, 0,
                  M3_EPI_NONE, nullptr, 0, q, nullptr, l == 0 ? &gp : nullptr, qs));
      Prod o;
      o.x = p_dqkv;
      o.res = p_hd;
      int p_hdo;
      if (attn) {
        // step j attends over the frame's codebook positions 0 .. j - 1
        const size_t lay = (size_t)B * c.d_heads * 8 * 128 * 2;
        o.x = ph;                                  // O reads the attention's output
        M3_TRY(attention(dqkv, d.dqkv, c.d_heads, c.d_heads, W,
                         reinterpret_cast<uint16_t*>(S + L.dkcache + l * lay),
                         reinterpret_cast<uint16_t*>(S + L.dvcache + l * lay), 8, j - 1, false,
                         ao, p_dqkv, tdao_slot(j, l), nullptr));
        p_hdo = ph;
        M3_TRY(gemv(c.fmt_depth, W.o, d.D, d.dq,
                    tagged ? reinterpret_cast<uint16_t*>(tdao_slot(j, l)) : ao, d.dq, nullptr, 0,
                    0, hd_o, d.D, 0, M3_EPI_RESIDUAL, hd, d.D, o));
      } else {
        p_hdo = ph;
        Sched os;
        os.follow = (d.dqkv + 15) / 16;
        M3_TRY(gemv(c.fmt_depth, W.o, d.D, d.dq, dqkv, d.dqkv, nullptr, 1, 2 * d.dq, hd_o, d.D, 0,
                    M3_EPI_RESIDUAL, hd, d.D, o, nullptr, nullptr, os));
      }
      Prod gu;
      gu.x = p_hdo;
      p_dmlp = ph;
      M3_TRY(gemv(c.fmt_depth, W.gate_up, 2 * d.Fd, d.D, hd_o, d.D, W.ffn_norm, 0, 0, dmlp, d.Fd,
                  0, M3_EPI_SWIGLU, nullptr, 0, gu));
      Prod dn;
      dn.x = p_dmlp;
      dn.res = p_hdo;
      p_hd = ph;
      M3_TRY(gemv(c.fmt_depth, W.down, d.D, d.Fd, dmlp, d.Fd, nullptr, 0, 0, hd_next, d.D, 0,
                  M3_EPI_RESIDUAL, hd_o, d.D, dn));
    }
    uint16_t* hd = hd_slot(j, c.d_layers);    // the step's output
    SampleEpi dep{c.seed, frame, (uint32_t)j, c.temperature, 0, 0, 0, part_dep(j), -1};
    Prod hp;
    hp.x = p_hd;
    p_dep = ph;
    M3_TRY(gemv(c.fmt_depth, m->heads[j - 1], d.CV, d.D, hd, d.D, m->d_final_norm, 0, 0, dlogits,
                d.CV, 1, M3_EPI_NONE, nullptr, 0, hp, guided ? nullptr : &dep));
    if (guided) {
      p_dep = ph;
      M3_TRY(guided_draw(dlogits, d.CV, d.CV, (uint32_t)j, 0, -1, part_dep(j)));
    }
  }
  // ---- last draw, feedback, code ring, frame counter ----
  FeedbackTags ft;
  if (tagged) {
    ft.last_part_prod = p_dep;
    ft.th = h_out;
    ft.th_prod = p_h;
    ft.h_out = h_plain_out;
    ft.seq = reinterpret_cast<uint32_t*>(S + L.seq);
  }
  ft.end_id = end_id;
  ft.stop = end_id >= 0 ? reinterpret_cast<uint32_t*>(S + L.stop) : nullptr;
  M3_TRY(sink.feedback(m->tok_emb_audio, m->audio_emb, codes, part_dep(d.ncb - 1),
                       guided ? 1 : n_blocks(d.CV),
                       c.vocab_base, c.n_slice, c.code_vocab, d.ncb, B, d.H, x, ring, frame, ft));
  return M3_OK;
}

// The persistent frame's steps as plain records of the memory each reads and
// writes (m3_frame_phase_table): byte ranges [lo, hi) with the producing
// step of what is read (-1: written before the launch or, for the frame end,
// earlier in the same launch) and whether the words carry tags.
struct RecordSink final : FrameSink {
  std::vector<m3_phase_record> recs;
  static m3_phase_region rows(const void* base, int B, size_t ld, size_t c0, size_t c1, size_t esz,
                              int producer, int tagged) {
    m3_phase_region r{};
    r.base = reinterpret_cast<uint64_t>(base);
    r.stride = ld * esz;
    r.rows = B;
    r.c0 = (uint32_t)(c0 * esz);
    r.c1 = (uint32_t)(c1 * esz);
    r.producer = producer;
    r.tagged = tagged;
    return r;
  }
  static void add(m3_phase_region* list, int32_t& n, const m3_phase_region& r) {
    if (n < M3_PHASE_MAX_REGIONS) list[n++] = r;
  }
  hipError_t gemv(const GemvDesc& d) override {
    m3_phase_record r{};
    r.kind = M3_PHASE_GEMV;
    const int B = d.B;
    if (d.gather) {
      const GatherPro& g = *d.gather;
      add(r.in, r.n_in, rows(g.u, B, d.K, 0, d.K, d.pu >= 0 ? 4 : 2, d.pu, d.pu >= 0));
      add(r.in, r.n_in, rows(g.part, B, g.nparts, 0, g.nparts, sizeof(Best), d.ppart, d.ppart >= 0));
      add(r.out, r.n_out, rows(g.out, B, d.K, 0, d.K, d.ytag ? 4 : 2, -1, d.ytag));
      add(r.out, r.n_out, rows(g.codes, B, 8, g.code_col, g.code_col + 1, 4, -1, 0));
    } else {
      // the attention stub reads the value heads only
      const size_t c0 = d.stub_group > 0 ? (size_t)d.stub_voff : 0;
      const size_t c1 = d.stub_group > 0 ? c0 + (size_t)d.K / d.stub_group : (size_t)d.K;
      add(r.in, r.n_in, rows(d.x, B, d.ldx, c0, c1, d.px >= 0 ? 4 : 2, d.px, d.px >= 0));
    }
    if (d.epi == M3_EPI_RESIDUAL)
      add(r.in, r.n_in, rows(d.res, B, d.ldr, 0, d.N, d.pres >= 0 ? 4 : 2, d.pres, d.pres >= 0));
    const size_t ncols = d.epi == M3_EPI_SWIGLU ? (size_t)d.N / 2 : (size_t)d.N;
    const size_t esz = d.out_f32 ? 4 : (d.ytag ? 4 : 2);
    add(r.out, r.n_out, rows(d.y, B, d.ldy, 0, ncols, esz, -1, d.out_f32 ? 0 : d.ytag));
    if (d.sample) {
      const int nb = n_blocks(d.N);
      add(r.out, r.n_out, rows(d.sample->part, B, nb, 0, nb, sizeof(Best), -1, d.ytag));
    }
    recs.push_back(r);
    return hipSuccess;
  }
  hipError_t cfg_draw(const CfgDesc& d) override {
    // the logits of the step before (it waits for every workgroup's flag of
    // that step), the one-entry winner record of each row
    m3_phase_record r{};
    r.kind = M3_PHASE_DRAW;
    add(r.in, r.n_in, rows(d.logits, 2 * d.S, d.ldl, 0, d.V, 4, (int)recs.size() - 1, 0));
    add(r.out, r.n_out, rows(d.part, 2 * d.S, 1, 0, 1, sizeof(Best), -1, 1));
    recs.push_back(r);
    return hipSuccess;
  }
  hipError_t attention(const AttnStep& s, int B) override {
    m3_phase_record r{};
    r.kind = M3_PHASE_ATTENTION;
    const size_t nqkv = (size_t)(s.n_q + 2 * s.n_kv) * 128, nq = (size_t)s.n_q * 128;
    add(r.in, r.n_in, rows(s.qkv, B, s.ldqkv, 0, nqkv, 4, s.pqkv, 1));
    // the caches ([row][KV head] sequences of max_pos rows of 128): a body
    // layer's whole cache (the frame's position is written and read back by
    // this step, the rest was written before the launch); a depth layer's
    // positions 0 .. pos (pos written here, the others by the layer's
    // attention at the frame's earlier codebook steps)
    const int seqs = B * s.n_kv;
    const size_t ld = (size_t)s.max_pos * 128;
    const size_t r0 = s.frame_dev ? 0 : (size_t)s.pos * 128;
    const size_t r1 = s.frame_dev ? ld : (size_t)(s.pos + 1) * 128;
    add(r.in, r.n_in, rows(s.k_cache, seqs, ld, 0, r1, 2, -1, 0));
    add(r.in, r.n_in, rows(s.v_cache, seqs, ld, 0, r1, 2, -1, 0));
    add(r.out, r.n_out, rows(s.k_cache, seqs, ld, r0, r1, 2, -1, 0));
    add(r.out, r.n_out, rows(s.v_cache, seqs, ld, r0, r1, 2, -1, 0));
    add(r.out, r.n_out, rows(s.tout, B, nq, 0, nq, 4, -1, 1));
    if (s.rec) {
      const size_t per = (size_t)s.n_q * body_attn_chunks_of(s, B) * (2 + 128);
      add(r.out, r.n_out, rows(s.rec, B, per, 0, per, 8, -1, 1));
    }
    recs.push_back(r);
    return hipSuccess;
  }
  hipError_t feedback(const uint16_t*, const uint16_t* const*, int32_t* codes, const Best* last_part,
                      int last_nparts, int32_t, int, int, int, int B, int H, uint16_t* x,
                      int32_t* ring, uint32_t* frame, const FeedbackTags& ft) override {
    m3_phase_record r{};
    r.kind = M3_PHASE_FRAME_END;
    add(r.in, r.n_in, rows(last_part, B, last_nparts, 0, last_nparts, sizeof(Best),
                           ft.last_part_prod, ft.last_part_prod >= 0));
    add(r.in, r.n_in, rows(ft.th, B, H, 0, H, ft.th_prod >= 0 ? 4 : 2, ft.th_prod, ft.th_prod >= 0));
    add(r.in, r.n_in, rows(codes, B, 8, 0, 7, 4, -1, 0));
    add(r.out, r.n_out, rows(x, B, H, 0, H, 2, -1, 0));
    add(r.out, r.n_out, rows(ft.h_out, B, H, 0, H, 2, -1, 0));
    add(r.out, r.n_out, rows(codes, B, 8, 7, 8, 4, -1, 0));
    add(r.out, r.n_out, rows(ring, 16 * B, 8, 0, 8, 4, -1, 0));
    (void)frame;
    recs.push_back(r);
    return hipSuccess;
  }
};

int enqueue_frame(const m3_model* m, uint8_t* S, int B, int32_t* codes, hipStream_t s) {
  LaunchSink sink(s);
  return build_frame(m, S, B, codes, sink);
}

// The depth decoder's part of a frame: every step before the depth input
// projection (the body's GEMVs and attention, the lm_head and the semantic
// draw; 4 GEMVs per body layer, then the lm_head) is dropped, the rest is
// launched as in the whole frame.
struct DepthOnlySink final : FrameSink {
  LaunchSink inner;
  int skip;                 // GEMVs still to drop
  bool sem_draw = true;     // a guided semantic draw (after the lm_head) still to drop
  DepthOnlySink(hipStream_t st, int n_skip) : inner(st), skip(n_skip) {}
  hipError_t gemv(const GemvDesc& d) override {
    if (skip > 0) {
      --skip;
      return hipSuccess;
    }
    return inner.gemv(d);
  }
  hipError_t cfg_draw(const CfgDesc& d) override {
    if (skip > 0) return hipSuccess;
    if (sem_draw) {
      sem_draw = false;
      return hipSuccess;
    }
    return inner.cfg_draw(d);
  }
  hipError_t attention(const AttnStep& a, int B) override {
    return skip > 0 ? hipSuccess : inner.attention(a, B);
  }
  hipError_t feedback(const uint16_t* tok, const uint16_t* const* aemb, int32_t* codes,
                      const Best* last_part, int last_nparts, int32_t vocab_base, int n_slice,
                      int code_vocab, int n_cb, int B, int H, uint16_t* x, int32_t* ring,
                      uint32_t* frame, const FeedbackTags& ft) override {
    return inner.feedback(tok, aemb, codes, last_part, last_nparts, vocab_base, n_slice, code_vocab,
                          n_cb, B, H, x, ring, frame, ft);
  }
};

int enqueue_depth(const m3_model* m, uint8_t* S, int B, int32_t* codes, hipStream_t s) {
  DepthOnlySink sink(s, 4 * m->cfg.n_layers + 1);
  return build_frame(m, S, B, codes, sink);
}

struct FrameGraph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

// the Gumbel-argmax draw's checks and launch (with a caller's workspace or
// the allocation-free scratch), defined after the entry points
int gumbel_check(const float* logits, int B, int V, int ldl, const m3_sample_params* p,
                 const int32_t* out);
int gumbel_entry(const float* logits, int B, int V, int ldl, const m3_sample_params* p,
                 int32_t* out, void* ws, size_t ws_bytes, void* stream);

}  // namespace

extern "C" {

const char* m3_status_str(int status) {
  switch (status) {
    case M3_OK: return "ok";
    case M3_ERR_NULL: return "a required pointer is NULL";
    case M3_ERR_SHAPE: return "a size is outside the supported set";
    case M3_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case M3_ERR_FORMAT: return "unknown weight format, epilogue or output type";
    case M3_ERR_WORKSPACE: return "workspace too small";
    case M3_ERR_HIP: return "a HIP call failed";
    case M3_ERR_ALIAS: return "an input overlaps an output";
    default: return "unknown status";
  }
}

const char* m3_version(void) { return "m3 0.1.0 gfx950"; }

size_t m3_packed_bytes(int fmt, int N, int K, int flags) {
  if (!fmt_ok(fmt) || N < 1 || !k_ok(fmt, K)) return 0;
  if (flags & ~M3_PACK_GLU_INTERLEAVE) return 0;
  if ((flags & M3_PACK_GLU_INTERLEAVE) && (N % 2) != 0) return 0;
  return (size_t)n_blocks(N) * block_bytes(fmt, K);
}

int m3_pack(int fmt, const uint16_t* W, int N, int K, int flags, void* packed, void* stream) {
  if (!W || !packed) return M3_ERR_NULL;
  if (!fmt_ok(fmt)) return M3_ERR_FORMAT;
  if (m3_packed_bytes(fmt, N, K, flags) == 0) return M3_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(packed, 16)) return M3_ERR_ALIGN;
  if (overlap(W, (size_t)N * K * 2, packed, m3_packed_bytes(fmt, N, K, flags))) return M3_ERR_ALIAS;
  return hip_status(launch_pack(fmt, W, N, K, flags, packed, static_cast<hipStream_t>(stream)));
}

int m3_rmsnorm_gemv(const void* w, int N, int K, const uint16_t* x, int B, int ldx,
                    const float* gamma, float eps, int stub_group, int stub_voff, void* y, int ldy,
                    int out_dtype, int epi, const uint16_t* res, int ldr, void* stream) {
  return gemv_entry(M3_BF16, w, N, K, x, B, ldx, gamma, eps, stub_group, stub_voff, y, ldy,
                    out_dtype, epi, res, ldr, stream);
}

int m3_gemv_i8row(const void* w, int N, int K, const uint16_t* x, int B, int ldx,
                  const float* gamma, float eps, int stub_group, int stub_voff, void* y, int ldy,
                  int out_dtype, int epi, const uint16_t* res, int ldr, void* stream) {
  return gemv_entry(M3_I8ROW, w, N, K, x, B, ldx, gamma, eps, stub_group, stub_voff, y, ldy,
                    out_dtype, epi, res, ldr, stream);
}

int m3_gemv_fp8row(const void* w, int N, int K, const uint16_t* x, int B, int ldx,
                   const float* gamma, float eps, int stub_group, int stub_voff, void* y, int ldy,
                   int out_dtype, int epi, const uint16_t* res, int ldr, void* stream) {
  return gemv_entry(M3_FP8ROW, w, N, K, x, B, ldx, gamma, eps, stub_group, stub_voff, y, ldy,
                    out_dtype, epi, res, ldr, stream);
}

int m3_gemv_i8g128(const void* w, int N, int K, const uint16_t* x, int B, int ldx,
                   const float* gamma, float eps, int stub_group, int stub_voff, void* y, int ldy,
                   int out_dtype, int epi, const uint16_t* res, int ldr, void* stream) {
  return gemv_entry(M3_I8G128, w, N, K, x, B, ldx, gamma, eps, stub_group, stub_voff, y, ldy,
                    out_dtype, epi, res, ldr, stream);
}

int m3_lmhead_sliced(int fmt, const void* packed_slice, int n_rows, int K, const uint16_t* x,
                     int B, int ldx, const float* gamma, float eps, float* logits, int ldl,
                     void* stream) {
  if (!row_fmt(fmt)) return M3_ERR_FORMAT;
  if (ldl % 4 != 0) return M3_ERR_ALIGN;
  const int st = validate_gemv(fmt, packed_slice, n_rows, K, x, B, ldx, gamma, eps, 0, 0, logits,
                               ldl, M3_OUT_F32, M3_EPI_NONE, nullptr, 0);
  if (st != M3_OK) return st;
  GemvDesc d{fmt, packed_slice, n_rows, K, x, ldx, B, gamma, eps, 0, 0, logits, ldl, 1,
             M3_EPI_NONE, nullptr, 0};
  return hip_status(launch_gemv(d, static_cast<hipStream_t>(stream)));
}

size_t m3_gumbel_workspace_bytes(int B, int V) {
  if (B < 1 || B > M3_MAX_B_SAMPLE || V < 1 || V > (1 << 24)) return 0;
  return sample_ws_bytes(B, V);
}

int m3_gumbel_argmax(const float* logits, int B, int V, int ldl, const m3_sample_params* p,
                     int32_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return M3_ERR_NULL;
  return gumbel_entry(logits, B, V, ldl, p, out, ws, ws_bytes, stream);
}

int m3_gumbel_argmax_noalloc(const float* logits, int B, int V, int ldl,
                             const m3_sample_params* p, int32_t* out, void* stream) {
  // every argument is checked before the scratch is looked up or anything runs
  const int st = gumbel_check(logits, B, V, ldl, p, out);
  if (st != M3_OK) return st;
  if (sample_ws_bytes(B, V) > kSampleScratchBytes) return M3_ERR_WORKSPACE;
  void* ws = nullptr;
  if (sample_scratch(&ws) != hipSuccess) return M3_ERR_HIP;
  return gumbel_entry(logits, B, V, ldl, p, out, ws, kSampleScratchBytes, stream);
}

}  // extern "C"

namespace {

int gumbel_check(const float* logits, int B, int V, int ldl, const m3_sample_params* p,
                 const int32_t* out) {
  if (!logits || !p || !out) return M3_ERR_NULL;
  if (B < 1 || B > M3_MAX_B_SAMPLE || V < 1 || V > (1 << 24) || ldl < V) return M3_ERR_SHAPE;
  if (!(p->temperature > 0.0f) || !std::isfinite(p->temperature)) return M3_ERR_SHAPE;
  if (!aligned(logits, 4) || !aligned(out, 4)) return M3_ERR_ALIGN;
  if ((p->ids && !aligned(p->ids, 4)) || (p->noise_override && !aligned(p->noise_override, 4)) ||
      (p->frame_dev && !aligned(p->frame_dev, 4)))
    return M3_ERR_ALIGN;
  return M3_OK;
}

int gumbel_entry(const float* logits, int B, int V, int ldl, const m3_sample_params* p,
                 int32_t* out, void* ws, size_t ws_bytes, void* stream) {
  const int st = gumbel_check(logits, B, V, ldl, p, out);
  if (st != M3_OK) return st;
  if (!aligned(ws, 16)) return M3_ERR_ALIGN;
  if (B < 1 || B > M3_MAX_B_SAMPLE || V < 1 || V > (1 << 24) || ldl < V) return M3_ERR_SHAPE;
  if (!(p->temperature > 0.0f) || !std::isfinite(p->temperature)) return M3_ERR_SHAPE;
  if (ws_bytes < sample_ws_bytes(B, V)) return M3_ERR_WORKSPACE;
  SampleDesc d{};
  d.logits = logits;
  d.B = B;
  d.V = V;
  d.ldl = ldl;
  d.seed = p->seed;
  d.frame = p->frame;
  d.frame_dev = p->frame_dev;
  d.draw = p->draw;
  d.temperature = p->temperature;
  d.index_base = p->index_base;
  d.ids = p->ids;
  d.valid_lo = p->valid_lo;
  d.valid_hi = p->valid_hi;
  d.noise = p->noise_override;
  d.out = out;
  d.out_stride = 1;
  d.ws = ws;
  return hip_status(launch_sample(d, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int m3_cfg_topk_draw(const float* logits, int n_songs, int V, int ldl, float cfg_scale,
                     int top_k, const m3_sample_params* p, int32_t* out, void* stream) {
  if (!logits || !p || !out) return M3_ERR_NULL;
  if (n_songs < 1 || n_songs > M3_MAX_SONGS_CFG || V < 1 || V > kCfgMaxV || ldl < V || top_k < 1)
    return M3_ERR_SHAPE;
  if (!std::isfinite(cfg_scale)) return M3_ERR_SHAPE;
  if (!(p->temperature > 0.0f) || !std::isfinite(p->temperature)) return M3_ERR_SHAPE;
  if (!aligned(logits, 4) || !aligned(out, 4)) return M3_ERR_ALIGN;
  if ((p->ids && !aligned(p->ids, 4)) || (p->noise_override && !aligned(p->noise_override, 4)) ||
      (p->frame_dev && !aligned(p->frame_dev, 4)))
    return M3_ERR_ALIGN;
  CfgDesc d{};
  d.logits = logits;
  d.S = n_songs;
  d.V = V;
  d.ldl = ldl;
  d.scale = cfg_scale;
  d.top_k = top_k;
  d.seed = p->seed;
  d.frame = p->frame;
  d.frame_dev = p->frame_dev;
  d.draw = p->draw;
  d.temperature = p->temperature;
  d.index_base = p->index_base;
  d.ids = p->ids;
  d.valid_lo = p->valid_lo;
  d.valid_hi = p->valid_hi;
  d.noise = p->noise_override;
  d.out = out;
  d.out_stride = 1;
  d.vec4 = aligned(logits, 16) && ldl % 4 == 0;
  return hip_status(launch_cfg_draw(d, static_cast<hipStream_t>(stream)));
}

int m3_rmsnorm_rows(const uint16_t* x, int M, int K, int ldx, const float* gamma, float eps,
                    uint16_t* a, int lda, void* stream) {
  if (!x || !gamma || !a) return M3_ERR_NULL;
  if (M < 1 || M > M3_MAX_M_PREFILL || K < 8 || K % 8 != 0 || ldx < K || lda < K) return M3_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return M3_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(a, 16) || !aligned(gamma, 16) || ldx % 8 || lda % 8)
    return M3_ERR_ALIGN;
  if (overlap(x, ((size_t)(M - 1) * ldx + K) * 2, a, ((size_t)(M - 1) * lda + K) * 2))
    return M3_ERR_ALIAS;
  return hip_status(
      launch_rmsnorm_rows(x, M, K, ldx, gamma, eps, a, lda, static_cast<hipStream_t>(stream)));
}

int m3_prefill_gemm(const void* w, int N, int K, const uint16_t* a, int M, int lda, void* y,
                    int ldy, int out_dtype, int epi, const uint16_t* res, int ldr, void* stream) {
  if (!w || !a || !y) return M3_ERR_NULL;
  if (out_dtype != M3_OUT_BF16 && out_dtype != M3_OUT_F32) return M3_ERR_FORMAT;
  if (epi != M3_EPI_NONE && epi != M3_EPI_SWIGLU && epi != M3_EPI_RESIDUAL) return M3_ERR_FORMAT;
  if (epi != M3_EPI_NONE && out_dtype != M3_OUT_BF16) return M3_ERR_FORMAT;
  if (epi == M3_EPI_RESIDUAL && !res) return M3_ERR_NULL;
  if (M < 1 || M > M3_MAX_M_PREFILL || N < 1 || K < 64 || K % 64 != 0 || lda < K) return M3_ERR_SHAPE;
  if (epi == M3_EPI_SWIGLU && N % 2 != 0) return M3_ERR_SHAPE;
  const int ncols = epi == M3_EPI_SWIGLU ? N / 2 : N;
  if (ldy < ncols || (epi == M3_EPI_RESIDUAL && ldr < N)) return M3_ERR_SHAPE;
  if ((size_t)n_blocks(N) * block_bytes(M3_BF16, K) >= ((size_t)1 << 31)) return M3_ERR_SHAPE;
  if (((size_t)(M - 1) * lda + K) * 2 >= ((size_t)1 << 31)) return M3_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(a, 16) || !aligned(y, 16) || lda % 8) return M3_ERR_ALIGN;
  const size_t esz = out_dtype == M3_OUT_F32 ? 4 : 2;
  if (overlap(a, ((size_t)(M - 1) * lda + K) * 2, y, ((size_t)(M - 1) * ldy + ncols) * esz))
    return M3_ERR_ALIAS;
  PrefillDesc d{w, N, K, a, M, lda, y, ldy, out_dtype == M3_OUT_F32, epi, res, ldr};
  return hip_status(launch_prefill_gemm(d, static_cast<hipStream_t>(stream)));
}

// ---- decode attention ------------------------------------------------------------
int m3_rope_table(float* table, int max_pos, int head_dim, float theta, void* stream) {
  if (!table) return M3_ERR_NULL;
  if (max_pos < 1 || max_pos > M3_MAX_POS || head_dim != M3_HEAD_DIM) return M3_ERR_SHAPE;
  if (!(theta > 1.0f) || !std::isfinite(theta)) return M3_ERR_SHAPE;
  if (!aligned(table, 16)) return M3_ERR_ALIGN;
  return hip_status(launch_rope_table(table, max_pos, head_dim, (double)theta,
                                      static_cast<hipStream_t>(stream)));
}

static bool attn_heads_ok(int n_q, int n_kv) {
  if (n_kv < 1 || n_q < n_kv || n_q % n_kv != 0 || n_q > M3_MAX_HEADS) return false;
  const int g = n_q / n_kv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

static size_t cache_bytes(int B, int n_kv, int max_pos) {
  return (size_t)B * n_kv * max_pos * M3_HEAD_DIM * 2;
}

int m3_qk_norm_rope(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv, int head_dim,
                    const float* q_gamma, const float* k_gamma, float eps, const float* rope,
                    int pos, uint16_t* q_out, int ldq, uint16_t* k_cache, uint16_t* v_cache,
                    int max_pos, void* stream) {
  if (!qkv || !q_gamma || !k_gamma || !rope || !q_out || !k_cache || !v_cache) return M3_ERR_NULL;
  if (head_dim != M3_HEAD_DIM || !attn_heads_ok(n_q, n_kv)) return M3_ERR_SHAPE;
  if (B < 1 || B > M3_MAX_B || max_pos < 1 || max_pos > M3_MAX_POS || pos < 0 || pos >= max_pos)
    return M3_ERR_SHAPE;
  if (ldqkv < (n_q + 2 * n_kv) * M3_HEAD_DIM || ldq < n_q * M3_HEAD_DIM) return M3_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return M3_ERR_SHAPE;
  if (!aligned(qkv, 16) || !aligned(q_out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(q_gamma, 4) || !aligned(k_gamma, 4) || !aligned(rope, 16) || ldqkv % 8 || ldq % 8)
    return M3_ERR_ALIGN;
  const size_t qkv_b = ((size_t)(B - 1) * ldqkv + (n_q + 2 * n_kv) * M3_HEAD_DIM) * 2;
  const size_t q_b = ((size_t)(B - 1) * ldq + n_q * M3_HEAD_DIM) * 2;
  const size_t c_b = cache_bytes(B, n_kv, max_pos);
  if (overlap(qkv, qkv_b, q_out, q_b) || overlap(qkv, qkv_b, k_cache, c_b) ||
      overlap(qkv, qkv_b, v_cache, c_b) || overlap(q_out, q_b, k_cache, c_b) ||
      overlap(q_out, q_b, v_cache, c_b) || overlap(k_cache, c_b, v_cache, c_b))
    return M3_ERR_ALIAS;
  return hip_status(launch_qk_norm_rope(qkv, B, ldqkv, n_q, n_kv, q_gamma, k_gamma, eps, rope, pos,
                                        q_out, ldq, k_cache, v_cache, max_pos,
                                        static_cast<hipStream_t>(stream)));
}

size_t m3_attention_workspace_bytes(int B, int n_q, int n_kv, int T) {
  if (B < 1 || B > M3_MAX_B || !attn_heads_ok(n_q, n_kv) || T < 1 || T > M3_MAX_POS) return 0;
  return attn_workspace_bytes(B, n_q, n_kv, T);
}

int m3_decode_attention(const uint16_t* q, int B, int ldq, int n_q, int n_kv, int head_dim,
                        const uint16_t* k_cache, const uint16_t* v_cache, int max_pos, int T,
                        uint16_t* out, int ldo, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!q || !k_cache || !v_cache || !out) return M3_ERR_NULL;
  if (head_dim != M3_HEAD_DIM || !attn_heads_ok(n_q, n_kv)) return M3_ERR_SHAPE;
  if (B < 1 || B > M3_MAX_B || max_pos < 1 || max_pos > M3_MAX_POS || T < 1 || T > max_pos)
    return M3_ERR_SHAPE;
  if (ldq < n_q * M3_HEAD_DIM || ldo < n_q * M3_HEAD_DIM) return M3_ERR_SHAPE;
  const size_t need = attn_workspace_bytes(B, n_q, n_kv, T);
  if (need && !workspace) return M3_ERR_NULL;
  if (workspace_bytes < need) return M3_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      (need && !aligned(workspace, 16)) || ldq % 8 || ldo % 8)
    return M3_ERR_ALIGN;
  const size_t q_b = ((size_t)(B - 1) * ldq + n_q * M3_HEAD_DIM) * 2;
  const size_t o_b = ((size_t)(B - 1) * ldo + n_q * M3_HEAD_DIM) * 2;
  const size_t c_b = cache_bytes(B, n_kv, max_pos);
  if (overlap(out, o_b, q, q_b) || overlap(out, o_b, k_cache, c_b) || overlap(out, o_b, v_cache, c_b) ||
      (need && (overlap(workspace, need, out, o_b) || overlap(workspace, need, q, q_b) ||
                overlap(workspace, need, k_cache, c_b) || overlap(workspace, need, v_cache, c_b))))
    return M3_ERR_ALIAS;
  return hip_status(launch_decode_attention(q, B, ldq, n_q, n_kv, k_cache, v_cache, max_pos, T, out,
                                            ldo, workspace, static_cast<hipStream_t>(stream)));
}

int m3_decode_attention_step(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                             int head_dim, const float* q_gamma, const float* k_gamma, float eps,
                             const float* rope, int pos, uint16_t* k_cache, uint16_t* v_cache,
                             int max_pos, uint16_t* out, int ldo, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!qkv || !q_gamma || !k_gamma || !rope || !k_cache || !v_cache || !out) return M3_ERR_NULL;
  if (head_dim != M3_HEAD_DIM || !attn_heads_ok(n_q, n_kv)) return M3_ERR_SHAPE;
  if (B < 1 || B > M3_MAX_B || max_pos < 1 || max_pos > M3_MAX_POS || pos < 0 || pos >= max_pos)
    return M3_ERR_SHAPE;
  if (ldqkv < (n_q + 2 * n_kv) * M3_HEAD_DIM || ldo < n_q * M3_HEAD_DIM) return M3_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return M3_ERR_SHAPE;
  const size_t need = attn_workspace_bytes(B, n_q, n_kv, pos + 1);
  if (need && !workspace) return M3_ERR_NULL;
  if (workspace_bytes < need) return M3_ERR_WORKSPACE;
  if (!aligned(qkv, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(q_gamma, 4) || !aligned(k_gamma, 4) || !aligned(rope, 16) ||
      (need && !aligned(workspace, 16)) || ldqkv % 8 || ldo % 8)
    return M3_ERR_ALIGN;
  const size_t qkv_b = ((size_t)(B - 1) * ldqkv + (n_q + 2 * n_kv) * M3_HEAD_DIM) * 2;
  const size_t o_b = ((size_t)(B - 1) * ldo + n_q * M3_HEAD_DIM) * 2;
  const size_t c_b = cache_bytes(B, n_kv, max_pos);
  if (overlap(qkv, qkv_b, out, o_b) || overlap(qkv, qkv_b, k_cache, c_b) ||
      overlap(qkv, qkv_b, v_cache, c_b) || overlap(out, o_b, k_cache, c_b) ||
      overlap(out, o_b, v_cache, c_b) || overlap(k_cache, c_b, v_cache, c_b) ||
      (need && (overlap(workspace, need, qkv, qkv_b) || overlap(workspace, need, out, o_b) ||
                overlap(workspace, need, k_cache, c_b) || overlap(workspace, need, v_cache, c_b))))
    return M3_ERR_ALIAS;
  return hip_status(launch_attention_fused(qkv, B, ldqkv, n_q, n_kv, q_gamma, k_gamma, eps, rope,
                                           pos, k_cache, v_cache, max_pos, out, ldo, workspace,
                                           static_cast<hipStream_t>(stream), nullptr, 0, nullptr));
}

// ---- the prompt's attention (S sequences of P positions, rows [s][t]) ------------
int m3_prefill_qk_norm_rope(const uint16_t* qkv, int S, int P, int ldqkv, int n_q, int n_kv,
                            int head_dim, const float* q_gamma, const float* k_gamma, float eps,
                            const float* rope, int pos_base, uint16_t* q_out, int ldq,
                            uint16_t* k_cache, uint16_t* v_cache, int max_pos, void* stream) {
  if (!qkv || !q_gamma || !k_gamma || !rope || !q_out || !k_cache || !v_cache) return M3_ERR_NULL;
  if (head_dim != M3_HEAD_DIM || !attn_heads_ok(n_q, n_kv)) return M3_ERR_SHAPE;
  if (S < 1 || S > M3_MAX_B || P < 1 || (long)S * P > M3_MAX_M_PREFILL || max_pos < 1 ||
      max_pos > M3_MAX_POS || pos_base < 0 || (long)pos_base + P > max_pos)
    return M3_ERR_SHAPE;
  if (ldqkv < (n_q + 2 * n_kv) * M3_HEAD_DIM || ldq < n_q * M3_HEAD_DIM) return M3_ERR_SHAPE;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return M3_ERR_SHAPE;
  if (!aligned(qkv, 16) || !aligned(q_out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(q_gamma, 4) || !aligned(k_gamma, 4) || !aligned(rope, 16) || ldqkv % 8 || ldq % 8)
    return M3_ERR_ALIGN;
  const int R = S * P;
  const size_t qkv_b = ((size_t)(R - 1) * ldqkv + (n_q + 2 * n_kv) * M3_HEAD_DIM) * 2;
  const size_t q_b = ((size_t)(R - 1) * ldq + n_q * M3_HEAD_DIM) * 2;
  const size_t c_b = cache_bytes(S, n_kv, max_pos);
  if (overlap(qkv, qkv_b, q_out, q_b) || overlap(qkv, qkv_b, k_cache, c_b) ||
      overlap(qkv, qkv_b, v_cache, c_b) || overlap(q_out, q_b, k_cache, c_b) ||
      overlap(q_out, q_b, v_cache, c_b) || overlap(k_cache, c_b, v_cache, c_b))
    return M3_ERR_ALIAS;
  return hip_status(launch_qk_norm_rope(qkv, R, ldqkv, n_q, n_kv, q_gamma, k_gamma, eps, rope,
                                        pos_base, q_out, ldq, k_cache, v_cache, max_pos,
                                        static_cast<hipStream_t>(stream), nullptr, 0, nullptr, P));
}

size_t m3_prefill_attention_workspace_bytes(int, int, int, int, int) {
  return 0;                                      // the tiled prompt kernel keeps no partial records
}

int m3_prefill_attention(const uint16_t* q, int S, int P, int ldq, int n_q, int n_kv, int head_dim,
                         const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                         int pos_base, uint16_t* out, int ldo, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !out) return M3_ERR_NULL;
  if (head_dim != M3_HEAD_DIM || !attn_heads_ok(n_q, n_kv)) return M3_ERR_SHAPE;
  if (S < 1 || S > M3_MAX_B || P < 1 || (long)S * P > M3_MAX_M_PREFILL || max_pos < 1 ||
      max_pos > M3_MAX_POS || pos_base < 0 || (long)pos_base + P > max_pos)
    return M3_ERR_SHAPE;
  if (ldq < n_q * M3_HEAD_DIM || ldo < n_q * M3_HEAD_DIM) return M3_ERR_SHAPE;
  const int R = S * P;
  (void)workspace;
  (void)workspace_bytes;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      ldq % 8 || ldo % 8)
    return M3_ERR_ALIGN;
  const size_t q_b = ((size_t)(R - 1) * ldq + n_q * M3_HEAD_DIM) * 2;
  const size_t o_b = ((size_t)(R - 1) * ldo + n_q * M3_HEAD_DIM) * 2;
  const size_t c_b = cache_bytes(S, n_kv, max_pos);
  if (overlap(out, o_b, q, q_b) || overlap(out, o_b, k_cache, c_b) || overlap(out, o_b, v_cache, c_b))
    return M3_ERR_ALIAS;
  // row (s, t) attends over positions 0 .. pos_base + t of sequence s
  return hip_status(launch_prompt_attention(q, S, P, ldq, n_q, n_kv, k_cache, v_cache, max_pos,
                                            pos_base, out, ldo, static_cast<hipStream_t>(stream)));
}

uint64_t m3_frame_weight_bytes(const m3_config* c) {
  if (!c) return 0;
  const Dims d = dims_of(*c);
  const int fb = c->fmt_body, fd = c->fmt_depth;
  const uint64_t layer = mat_bytes(fb, d.nqkv, d.H) + mat_bytes(fb, d.H, d.nq) +
                         mat_bytes(fb, 2ull * d.F, d.H) + mat_bytes(fb, d.H, d.F);
  uint64_t total = (uint64_t)c->n_layers * layer + 4ull * d.H * (2ull * c->n_layers + 1);
  total += mat_bytes(c->fmt_lm, d.VL, d.H);
  total += mat_bytes(fd, d.D, d.H);
  const uint64_t dlayer = mat_bytes(fd, d.dqkv, d.D) + mat_bytes(fd, d.D, d.dq) +
                          mat_bytes(fd, 2ull * d.Fd, d.D) + mat_bytes(fd, d.D, d.Fd);
  const uint64_t step = (uint64_t)c->d_layers * dlayer + mat_bytes(fd, d.CV, d.D) +
                        4ull * d.D * (2ull * c->d_layers + 1);
  total += (uint64_t)(d.ncb - 1) * step;
  return total;
}

int m3_frame_layout_get(const m3_config* cfg, int B, m3_frame_layout* out) {
  if (!out) return M3_ERR_NULL;
  const int st = validate_config(cfg, B);
  if (st != M3_OK) return st;
  *out = layout_of(*cfg, B);
  return M3_OK;
}

size_t m3_frame_workspace_bytes(const m3_config* cfg, int B) {
  if (validate_config(cfg, B) != M3_OK) return 0;
  return layout_of(*cfg, B).total;
}

int m3_frame_state_init(const m3_config* cfg, int B, void* state, const uint16_t* x0,
                        uint32_t frame0, void* stream) {
  if (!state || !x0) return M3_ERR_NULL;
  const int st = validate_config(cfg, B);
  if (st != M3_OK) return st;
  if (!aligned(state, 256) || !aligned(x0, 16)) return M3_ERR_ALIGN;
  const m3_frame_layout L = layout_of(*cfg, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* S = static_cast<uint8_t*>(state);
  M3_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(S), 0u, L.total / 4, s));
  M3_TRY(launch_copy_bf16(x0, reinterpret_cast<uint16_t*>(S + L.x), (size_t)B * cfg->hidden, s));
  M3_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(S + L.frame), frame0, 1, s));
  if (cfg->attention)
    M3_TRY(launch_rope_table(reinterpret_cast<float*>(S + L.rope), std::max(cfg->max_pos, 8), 128,
                             1e6, s));
  // (flags, error word, launch counter, tagged streams and caches start at zero)
  return M3_OK;
}

int m3_decode_frame_weights(const m3_model* model, void* state, int B, int32_t* codes,
                            uint64_t* bytes_read, void* stream) {
  if (!model || !state || !codes) return M3_ERR_NULL;
  int st = validate_config(&model->cfg, B);
  if (st != M3_OK) return st;
  st = validate_model(model);
  if (st != M3_OK) return st;
  if (!aligned(state, 256) || !aligned(codes, 16)) return M3_ERR_ALIGN;
  if (bytes_read) *bytes_read = m3_frame_weight_bytes(&model->cfg);
  return enqueue_frame(model, static_cast<uint8_t*>(state), B, codes,
                       static_cast<hipStream_t>(stream));
}

namespace {
int graph_create(const m3_model* model, void* state, int B, int32_t* codes, void* stream,
                 void** graph_out, bool depth_only) {
  if (!model || !state || !codes || !graph_out) return M3_ERR_NULL;
  int st = validate_config(&model->cfg, B);
  if (st != M3_OK) return st;
  st = validate_model(model);
  if (st != M3_OK) return st;
  if (!aligned(state, 256) || !aligned(codes, 16)) return M3_ERR_ALIGN;
  if (!stream) return M3_ERR_NULL;   // the legacy default stream cannot be captured
  M3_TRY(gemv_prepare());
  hipStream_t s = static_cast<hipStream_t>(stream);
  M3_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
  const int est = depth_only ? enqueue_depth(model, static_cast<uint8_t*>(state), B, codes, s)
                             : enqueue_frame(model, static_cast<uint8_t*>(state), B, codes, s);
  hipGraph_t g = nullptr;
  const hipError_t ce = hipStreamEndCapture(s, &g);
  if (est != M3_OK || ce != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return est != M3_OK ? est : M3_ERR_HIP;
  }
  hipGraphExec_t ex = nullptr;
  if (hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return M3_ERR_HIP;
  }
  FrameGraph* fg = new (std::nothrow) FrameGraph{g, ex};
  if (!fg) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return M3_ERR_HIP;
  }
  *graph_out = fg;
  return M3_OK;
}
}  // namespace

int m3_frame_graph_create(const m3_model* model, void* state, int B, int32_t* codes, void* stream,
                          void** graph_out) {
  return graph_create(model, state, B, codes, stream, graph_out, false);
}

int m3_depth_graph_create(const m3_model* model, void* state, int B, int32_t* codes, void* stream,
                          void** graph_out) {
  return graph_create(model, state, B, codes, stream, graph_out, true);
}

int m3_frame_graph_launch(void* graph, void* stream) {
  if (!graph) return M3_ERR_NULL;
  FrameGraph* fg = static_cast<FrameGraph*>(graph);
  return hip_status(hipGraphLaunch(fg->exec, static_cast<hipStream_t>(stream)));
}

int m3_frame_graph_destroy(void* graph) {
  if (!graph) return M3_ERR_NULL;
  FrameGraph* fg = static_cast<FrameGraph*>(graph);
  const hipError_t a = hipGraphExecDestroy(fg->exec);
  const hipError_t b = hipGraphDestroy(fg->graph);
  delete fg;
  return (a == hipSuccess && b == hipSuccess) ? M3_OK : M3_ERR_HIP;
}

int m3_frame_persistent_create(const m3_model* model, void* state, int B, int32_t* codes,
                               void* stream, void** handle_out) {
  if (!model || !state || !codes || !handle_out) return M3_ERR_NULL;
  int st = validate_config(&model->cfg, B);
  if (st != M3_OK) return st;
  st = validate_model(model);
  if (st != M3_OK) return st;
  if (!aligned(state, 256) || !aligned(codes, 16)) return M3_ERR_ALIGN;
  if (frame_phases(model->cfg) > persist_max_phases()) return M3_ERR_SHAPE;
  // one frame kernel per body format: bf16, int8-row or fp8-row body and the
  // same lm_head format, int8-g128 depth
  const m3_config& c = model->cfg;
  if (!row_fmt(c.fmt_body) || c.fmt_lm != c.fmt_body || c.fmt_depth != M3_I8G128)
    return M3_ERR_FORMAT;
  // row-block winners carry their column in 16 bits next to the tag
  if (c.n_slice + 1 > 65535 || c.code_vocab > 65535) return M3_ERR_SHAPE;
  uint8_t* S = static_cast<uint8_t*>(state);
  const m3_frame_layout L = layout_of(model->cfg, B);
  PersistPlan* pl = persist_plan_new(B);
  if (!pl) return M3_ERR_HIP;
  PlanSink sink(pl);
  st = build_frame(model, S, B, codes, sink, true);
  // recording makes no HIP call: a failure is a step the frame kernel does not carry
  if (st == M3_ERR_HIP) st = M3_ERR_SHAPE;
  if (st == M3_OK && persist_plan_size(pl) != frame_phases(model->cfg)) st = M3_ERR_SHAPE;
  PersistLaunch* PL = st == M3_OK ? persist_launch_new() : nullptr;
  if (st == M3_OK && PL) {
    const hipError_t e = persist_upload(pl, S + L.phases, reinterpret_cast<uint32_t*>(S + L.flags),
                                        reinterpret_cast<uint32_t*>(S + L.err),
                                        reinterpret_cast<uint32_t*>(S + L.seq),
                                        static_cast<hipStream_t>(stream), PL);
    if (e != hipSuccess) st = M3_ERR_HIP;
  } else if (st == M3_OK) {
    st = M3_ERR_HIP;
  }
  persist_plan_free(pl);
  if (st != M3_OK) {
    if (PL) persist_launch_free(PL);
    return st;
  }
  *handle_out = PL;
  return M3_OK;
}

int m3_frame_phase_table(const m3_model* model, void* state, int B, int32_t* codes,
                         m3_phase_record* out, int max_records) {
  if (!model || !state || !codes) return M3_ERR_NULL;
  int st = validate_config(&model->cfg, B);
  if (st != M3_OK) return st;
  st = validate_model(model);
  if (st != M3_OK) return st;
  const m3_config& c = model->cfg;
  RecordSink sink;
  st = build_frame(model, static_cast<uint8_t*>(state), B, codes, sink, true);
  if (st == M3_ERR_HIP) st = M3_ERR_SHAPE;
  if (st != M3_OK) return st;
  const int n = (int)sink.recs.size();
  if (out) {
    if (max_records < n) return M3_ERR_WORKSPACE;
    for (int i = 0; i < n; ++i) out[i] = sink.recs[i];
  }
  return n;
}

int m3_frame_persistent_launch(void* handle, void* stream) {
  if (!handle) return M3_ERR_NULL;
  return hip_status(persist_launch(*static_cast<PersistLaunch*>(handle),
                                   static_cast<hipStream_t>(stream)));
}

int m3_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, int nontemporal,
                   void* stream) {
  if (!buf || !sink) return M3_ERR_NULL;
  if (bytes < 16 || bytes % 16 || bytes >= ((size_t)1 << 31) || workgroups < 1 || workgroups > 4096)
    return M3_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return M3_ERR_ALIGN;
  return hip_status(launch_stream_read(buf, bytes, sink, workgroups, nontemporal,
                                       static_cast<hipStream_t>(stream)));
}

size_t m3_frame_persistent_clock_bytes(void* handle) {
  if (!handle) return 0;
  return persist_clock_words(*static_cast<PersistLaunch*>(handle)) * 8;
}

int m3_frame_persistent_clock(void* handle, uint64_t* clk, size_t clk_bytes, int* n_phases,
                              int* n_workgroups) {
  if (!handle) return M3_ERR_NULL;
  PersistLaunch& PL = *static_cast<PersistLaunch*>(handle);
  int nwg = 0;
  const int nph = persist_launch_dims(PL, &nwg);
  if (n_phases) *n_phases = nph;
  if (n_workgroups) *n_workgroups = nwg;
  if (clk) {
    if (!aligned(clk, 8)) return M3_ERR_ALIGN;
    if (clk_bytes < persist_clock_words(PL) * 8) return M3_ERR_WORKSPACE;
  }
  persist_set_clock(PL, clk);
  return M3_OK;
}

int m3_frame_persistent_destroy(void* handle) {
  if (!handle) return M3_ERR_NULL;
  persist_launch_free(static_cast<PersistLaunch*>(handle));
  return M3_OK;
}

}  // extern "C"
