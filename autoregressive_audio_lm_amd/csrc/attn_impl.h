#pragma once
// attn_impl.h -- device code of decode attention shared by the standalone
// kernels (attention.hip) and the persistent frame's attention phases
// (persist_kernel.h), so that both compute the same bits: one head's q/k
// RMSNorm + RoPE, and the attention of one row's G query heads over one chunk
// of cached positions (the partial softmax of "MiniMax Music 3, local" and
// TensorFold PR #987's split-key decode attention; fp32 scores, softmax and
// sums over bf16 operands).
//
// A chunk is worked by 256 threads (4 waves).  Pass 1: four lanes per
// position, each holding 32 of the 128 dimensions as bf16 pairs; v_dot2
// products against the G query heads, a two-step DPP sum, the scores (base 2,
// scale folded in) to LDS.  One wave per head then takes the chunk's maximum,
// exponentials and sum.  Pass 2: each lane owns 4 dimensions of CH / 8
// positions (a wave load reads two whole value rows) and accumulates P.V; the
// 8 half-wave partials are summed in LDS in a fixed order.
#include "gemv_impl.h"

namespace m3 {

constexpr int kHD = 128;
constexpr int kAThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// One head's RMSNorm + RoPE (lane l holds elements l and l + 64 as raw bf16
// bits; every lane of the wave takes part): the GEMV prologue's norm steps
// (float64 sum of squares, r rounded once to fp32, two fp32 products, one bf16
// rounding), then the rotation of the pair (l, l + 64) by the position's
// angle from the table, rounded to bf16.
__device__ __forceinline__ void head_norm_rope(uint32_t x0, uint32_t x1, const float* g, float eps,
                                               const float* rope, int pos, int lane, uint32_t& y0,
                                               uint32_t& y1) {
  const float a0f = bf2f(x0), a1f = bf2f(x1);
  const float r = norm_r(wave_sum_f64((double)a0f * a0f + (double)a1f * a1f), kHD, eps);
  const float a0 = bf2f(f2bf((a0f * r) * g[lane])), a1 = bf2f(f2bf((a1f * r) * g[lane + 64]));
  const float c = rope[((size_t)pos * 64 + lane) * 2], s = rope[((size_t)pos * 64 + lane) * 2 + 1];
  y0 = f2bf(a0 * c - a1 * s);
  y1 = f2bf(a1 * c + a0 * s);
}

template <int G, int CH>
struct AttnLds {
  float S[CH][G];                       // scores, then probabilities
  float Ms[G], Ls[G];
  alignas(16) float pacc[8][G][kHD];    // P.V partials of the 8 half-waves
};

template <int G, int CH>
struct AttnRegs {
  static constexpr int PJ = CH / 64;    // pass-1 positions per 4-lane group
  static constexpr int PI = CH / 8;     // pass-2 positions per lane
  static constexpr int WP = CH / 4;     // pass-2 positions per wave
  uint4 qr[G][4];
  uint4 kr[PJ][4];
  uint2 vr[PI];
};

// q of the G heads: contiguous 128-element bf16 rows at q (global or LDS).
// Pass-1 layout: a group of 4 lanes per position, lane li holding the 16-byte
// chunks 4 c + li (c < 4) of a row.
template <int G, int CH>
__device__ __forceinline__ void attn_load_q(AttnRegs<G, CH>& R, const uint16_t* q, int tid) {
  const int li = tid & 3;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      R.qr[h][c] = *reinterpret_cast<const uint4*>(q + (size_t)h * kHD + 8 * (4 * c + li));
}

// position of the pass-1 row j of this lane's group and of the pass-2 row i
// of this lane, within positions t0 .. t0 + n - 1 (rows past n repeat the last)
template <int G, int CH>
__device__ __forceinline__ int attn_kpos(int t0, int n, int tid, int j) {
  return t0 + min((tid >> 2) + 64 * j, n - 1);
}
template <int G, int CH>
__device__ __forceinline__ int attn_vpos(int t0, int n, int tid, int i) {
  return t0 + min(AttnRegs<G, CH>::WP * (tid >> 6) + 2 * i + ((tid & 63) >> 5), n - 1);
}

// keys and values of positions t0 .. t0 + n - 1 (kb, vb: the KV head's rows
// of 128 bf16 from position 0).  Pass-2 layout: the lane owns dimensions
// 4 dq .. 4 dq + 3 of positions WP w + 2 i + sub.
template <int G, int CH>
__device__ __forceinline__ void attn_load_kv(AttnRegs<G, CH>& R, const uint16_t* kb,
                                             const uint16_t* vb, int t0, int n, int tid) {
  const int li = tid & 3, dq = tid & 31;
#pragma unroll
  for (int j = 0; j < AttnRegs<G, CH>::PJ; ++j) {
    const int t = attn_kpos<G, CH>(t0, n, tid, j);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      R.kr[j][c] = *reinterpret_cast<const uint4*>(kb + (size_t)t * kHD + 8 * (4 * c + li));
  }
#pragma unroll
  for (int i = 0; i < AttnRegs<G, CH>::PI; ++i) {
    const int t = attn_vpos<G, CH>(t0, n, tid, i);
    R.vr[i] = *reinterpret_cast<const uint2*>(vb + (size_t)t * kHD + 4 * dq);
  }
}

// the key and value rows of position tn taken from krow, vrow (128 bf16
// each; the rows attn_load_kv requested were written after the request)
template <int G, int CH>
__device__ __forceinline__ void attn_set_kv_at(AttnRegs<G, CH>& R, const uint16_t* krow,
                                               const uint16_t* vrow, int t0, int n, int tid,
                                               int tn) {
  const int li = tid & 3, dq = tid & 31;
#pragma unroll
  for (int j = 0; j < AttnRegs<G, CH>::PJ; ++j) {
    if (attn_kpos<G, CH>(t0, n, tid, j) != tn) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      R.kr[j][c] = *reinterpret_cast<const uint4*>(krow + 8 * (4 * c + li));
  }
#pragma unroll
  for (int i = 0; i < AttnRegs<G, CH>::PI; ++i)
    if (attn_vpos<G, CH>(t0, n, tid, i) == tn)
      R.vr[i] = *reinterpret_cast<const uint2*>(vrow + 4 * dq);
}

// The chunk's n positions (1 <= n <= CH) against the G heads.  out(h, d, A,
// M, L) receives, for every head h and dimension d, the chunk's P.V sum A,
// maximum score M (base 2) and sum of exponentials L.  The 256 threads (tid
// 0 .. 255) pass three workgroup barriers.  q: nullptr to take the heads
// from R.qr (attn_load_q), or their rows in LDS, read where pass 1 needs
// them (fewer registers; the same products in the same order).
template <int G, int CH, class Out>
__device__ __forceinline__ void attn_compute(const AttnRegs<G, CH>& R, int n, float scale2, int tid,
                                             AttnLds<G, CH>& L, Out&& out,
                                             const uint16_t* q = nullptr) {
  constexpr int PJ = AttnRegs<G, CH>::PJ, PI = AttnRegs<G, CH>::PI, WP = AttnRegs<G, CH>::WP;
  const int lane = tid & 63, wave = tid >> 6, grp = tid >> 2, li = tid & 3;
  // pass 1: scores (base 2, scale folded in); masked positions get -inf
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int tc = grp + 64 * j;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 qv = q ? *reinterpret_cast<const uint4*>(q + (size_t)h * kHD + 8 * (4 * c + li))
                           : R.qr[h][c];
        s = dot2(qv.x, R.kr[j][c].x, s);
        s = dot2(qv.y, R.kr[j][c].y, s);
        s = dot2(qv.z, R.kr[j][c].z, s);
        s = dot2(qv.w, R.kr[j][c].w, s);
      }
      s += dpp_f<0xB1>(s);                       // the 4 lanes of the group
      s += dpp_f<0x4E>(s);
      if (li == 0) L.S[tc][h] = tc < n ? s * scale2 : -INFINITY;
    }
  }
  __syncthreads();
  // softmax over the chunk, one wave per head
  for (int h = wave; h < G; h += 4) {
    float e[PJ], m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PJ; ++j) m = fmaxf(m, L.S[lane + 64 * j][h]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      e[j] = exp2f(L.S[lane + 64 * j][h] - m);
      L.S[lane + 64 * j][h] = e[j];
      l += e[j];
    }
    l = wave_sum(l);
    if (lane == 0) {
      L.Ms[h] = m;
      L.Ls[h] = l;
    }
  }
  __syncthreads();
  // pass 2: P.V over this lane's positions and 4 dimensions
  const int dq = lane & 31, sub = lane >> 5;
  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < PI; ++i) {
    const int tc = WP * wave + 2 * i + sub;
    const float v0 = bf2f(R.vr[i].x & 0xffffu), v1 = bf2f(R.vr[i].x >> 16);
    const float v2 = bf2f(R.vr[i].y & 0xffffu), v3 = bf2f(R.vr[i].y >> 16);
    float prs[G];                                // 0 for masked positions
#pragma unroll
    for (int h = 0; h < G; ++h) prs[h] = L.S[tc][h];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = prs[h];
      acc[h][0] = fmaf(pr, v0, acc[h][0]);
      acc[h][1] = fmaf(pr, v1, acc[h][1]);
      acc[h][2] = fmaf(pr, v2, acc[h][2]);
      acc[h][3] = fmaf(pr, v3, acc[h][3]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
    *reinterpret_cast<float4*>(&L.pacc[2 * wave + sub][h][4 * dq]) =
        make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  __syncthreads();
  for (int o = tid; o < G * kHD; o += kAThreads) {
    const int h = o / kHD, d = o % kHD;
    float A = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) A += L.pacc[k][h][d];
    out(h, d, A, L.Ms[h], L.Ls[h]);
  }
}

}  // namespace m3
