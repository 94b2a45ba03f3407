#pragma once
// frame_impl.h -- the end of a decode frame: the last codebook's draw, the
// frame-embedding feedback, the 16-frame code ring and the GPU-side frame
// counter.  Shared by the one-launch kernel (frame.hip) and the persistent
// frame kernel (persist.hip); COH selects the system-coherent accesses the
// persistent launch needs (see gemv_impl.h).
//
// DiffSynth-Studio MiniMax-Music3 article, stage 2: after the semantic code,
// the RVQ depth decoder draws the remaining 7 codes one codebook at a time;
// the frame's 8 codes are embedded (embed_tokens of the semantic id plus the
// RVQ audio embeddings of the 7 residual codes), scaled by 8^-1/2 and fed back
// as the next frame's input.  TensorFold PR #987: position and count advance
// on the GPU; the host reads the drawn tokens every 16 frames.
#include "gemv_impl.h"

namespace m3 {
namespace {

struct FeedbackArgs {
  const uint16_t* tok;           // [n_slice, H]
  const uint16_t* aemb[8];       // [code_vocab, H] for codebooks 1..n_cb-1
  int32_t* codes;                // [B, 8]
  const Best* last_part;         // [B, last_nparts] winners of the last head's row blocks
  int last_nparts;
  int32_t vocab_base;
  int n_slice, code_vocab, n_cb, B, H;
  uint16_t* x;
  int32_t* ring;                 // [16, B, 8]
  uint32_t* frame;
  // persistent launch: the last head's winners and the tagged body stream
  // (plain copy into h_out), the phases that wrote them, the launch counter
  int last_part_prod;            // -1: plain winners
  const void* th;                // tagged [B, H] or nullptr
  int th_prod;
  uint16_t* h_out;
  uint32_t* seq;                 // nullptr: no launch counter
  int32_t end_id;                // >= 0: the end token's id
  uint32_t* stop;                // [B] stop words (nullptr: no end token)
};

// the last codebook's draw for row b, by one wave (same total order as the sampler)
template <bool COH>
__device__ int last_code(const FeedbackArgs& a, int b, uint32_t ebase) {
  const int lane = threadIdx.x & 63;
  const uint32_t tag = tag_of(a.last_part_prod, ebase);
  float bz = -INFINITY;
  int bj = 0x7fffffff;
  for (int c = lane; c < a.last_nparts; c += 64) {
    const Best r = part_load<COH>(a.last_part, (size_t)b * a.last_nparts + c, tag, nullptr);
    if (above(r.z, r.j, bz, bj)) {
      bz = r.z;
      bj = r.j;
    }
  }
  best_reduce(bz, bj, 64);
  return __shfl(bj, 0, 64);
}

// Workgroup wg of nwg (nthreads threads) embeds rows b = wg, wg + nwg, ...;
// workgroup 0 also writes every row's last code, the ring slot of this frame
// and advances the frame counter (it is the counter's only reader here).
// c_last: LDS scratch of M3_MAX_B_FRAME ints.
// (persistent launch: every workgroup has published its last phase before
// this runs, so the tagged inputs are complete and nothing here waits)
template <bool COH>
__device__ __forceinline__ void feedback_run(const FeedbackArgs& a, int wg, int nwg, int* c_last, uint32_t ebase) {
  const int nthreads = blockDim.x, nwave = nthreads >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool leader = wg == 0;
  for (int b = wave; b < a.B; b += nwave) {
    if (leader || b % nwg == wg) {
      const int c = last_code<COH>(a, b, ebase);
      if (lane == 0) c_last[b] = c;
    }
  }
  __syncthreads();
  const float sc = 1.0f / sqrtf((float)a.n_cb);
  for (int b = wg; b < a.B; b += nwg) {
    int c0 = (int)ld4<COH>(a.codes, (size_t)b * 8 * 4) - a.vocab_base;
    if (c0 < 0 || c0 >= a.n_slice) c0 = 0;
    // (loops over codebooks fully unrolled: register arrays, no scratch)
    int cs[8];
#pragma unroll
    for (int cb = 1; cb < 8; ++cb) {
      int c = 0;
      if (cb < a.n_cb) c = cb == a.n_cb - 1 ? c_last[b] : (int)ld4<COH>(a.codes, (size_t)(b * 8 + cb) * 4);
      cs[cb] = (c < 0 || c >= a.code_vocab) ? 0 : c;
    }
    for (int k = threadIdx.x * 8; k < a.H; k += nthreads * 8) {
      float acc[8];
      const uint4 t = *reinterpret_cast<const uint4*>(a.tok + (size_t)c0 * a.H + k);
      const uint32_t tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = bf2f(tv[j] & 0xffffu);
        acc[2 * j + 1] = bf2f(tv[j] >> 16);
      }
#pragma unroll
      for (int cb = 1; cb < 8; ++cb) {
        if (cb >= a.n_cb) break;
        const uint4 v = *reinterpret_cast<const uint4*>(a.aemb[cb - 1] + (size_t)cs[cb] * a.H + k);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += bf2f(vv[j] & 0xffffu);
          acc[2 * j + 1] += bf2f(vv[j] >> 16);
        }
      }
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f2bf(acc[2 * j] * sc) | (f2bf(acc[2 * j + 1] * sc) << 16);
      st16<COH>(a.x, ((size_t)b * a.H + k) * 2, make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
  if (COH && a.th) {
    // plain copy of the body's final residual stream for the caller
    const uint32_t tag = tag_of(a.th_prod, ebase);
    for (int b = wg; b < a.B; b += nwg)
      for (int k = threadIdx.x * 8; k < a.H; k += nthreads * 8)
        st16<COH>(a.h_out, ((size_t)b * a.H + k) * 2,
                  act_load8<COH>(a.th, (size_t)b * a.H + k, tag, nullptr));
  }
  if (leader) {
    const uint32_t f = ld4<COH>(a.frame, 0);
    // a row's first end token: its stop word becomes the frame number + 1
    if (a.stop)
      for (int b = threadIdx.x; b < a.B; b += nthreads)
        if ((int32_t)ld4<COH>(a.codes, (size_t)b * 8 * 4) == a.end_id &&
            ld4<COH>(a.stop, (size_t)b * 4) == 0u)
          st4<COH>(a.stop, (size_t)b * 4, f + 1u);
    for (int i = threadIdx.x; i < a.B * 8; i += nthreads) {
      const int b = i >> 3, cb = i & 7;
      const int32_t v = cb == a.n_cb - 1 ? c_last[b] : (int32_t)ld4<COH>(a.codes, (size_t)i * 4);
      if (cb == a.n_cb - 1) st4<COH>(a.codes, (size_t)i * 4, (uint32_t)v);
      st4<COH>(a.ring, ((size_t)(f & 15u) * a.B * 8 + i) * 4, (uint32_t)v);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      st4<COH>(a.frame, 0, f + 1u);
      if (a.seq) st4<COH>(a.seq, 0, ld4<COH>(a.seq, 0) + 1u);
    }
  }
}

}  // namespace
}  // namespace m3
