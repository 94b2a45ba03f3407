#pragma once
// persist_attn.h -- the persistent frame's attention phases: decode attention
// in place of the identity stub, for a body layer at the frame's position or
// for a depth layer at the codebook step's position, inside the one launch
// that runs the whole frame (see persist.hip).
//
// One phase does what the graph frame does in three launches (q/k norm +
// RoPE with the cache write, the chunks' partial softmax, the merge), with
// the same arithmetic (attn_impl.h), so the two frames produce the same bits:
//  - chunk items (row, KV head, chunk of CH positions): the item first
//    requests its chunk's cached keys and values, then waits for the QKV
//    words it needs (tagged, like every GEMV operand of the launch), norms and
//    rotates its G query heads into LDS and, for the chunk holding the
//    frame's position, writes that position's key and value to the cache and
//    uses them from LDS; a workgroup runs two items at once, one per 256-thread
//    half.  A single chunk writes the output words; otherwise each item
//    leaves (maximum, sum, P.V) as tagged 64-bit records.
//  - merge items (row, query head), four per workgroup, on the workgroups
//    counted from the last: each waits for its head's records and combines
//    them in chunk order, as the merge kernel does, into the output words.
// A workgroup finishes its chunk items before it starts a merge, so every
// record a merge waits for is produced.  The output words are the O GEMV's
// operand, tagged with this phase.
//
// Cache visibility.  The chunk holding position pos is worked by the
// workgroup that writes pos, which takes that row from LDS; every other
// cached row was written before the launch, except in
// the depth decoder, whose step j writes position j - 1 of a per-layer cache
// that steps j + 1 .. 7 read: item (row, head) goes to the same workgroup at
// every step, so these rows too are read by the workgroup that wrote them.
#include "attn_impl.h"

namespace m3 {

// (AttnArgs, the phase's parameters, is in m3_internal.h: it is stored in the
// phase table in place of a GEMV's Params.)

// LDS of an attention phase, per half: an AttnLds, G rotated q rows and the
// key and value rows of the frame's position
template <int G, int CH>
constexpr size_t attn_phase_smem() {
  return 2 * sizeof(AttnLds<G, CH>) + 2 * (size_t)(G + 2) * kHD * 2;
}

// a chunk record value: the float's bits with the 16-bit tag above them
__device__ __forceinline__ void rec_store(uint64_t* p, float v, uint32_t tag) {
  M3_COH_STORE(p, (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32));
}
__device__ __forceinline__ float rec_load(const uint64_t* p, uint32_t tag, uint32_t* err) {
  uint64_t v = M3_COH_LOAD(p);
  long n = 0;
  while ((uint32_t)(v >> 32) != tag && spin_more(n, err)) v = M3_COH_LOAD(p);
  return __uint_as_float((uint32_t)v);
}

// One (row b, query head qh) merge by 128 threads (d = dimension): chunk c's
// maximum and sum are held by lane c % 64; the maximum over all chunks, then
// L = sum l_c e_c and A = sum a_c e_c with e_c = 2^(m_c - M), accumulated in
// chunk order with the merge kernel's fused multiply-adds.  Each lane first
// waits for its chunk's maximum; the sums and this thread's values of up to
// kBatch chunks are then requested at once (by then the records are, as a
// rule, complete, so they come back in one round trip).
template <int G>
__device__ __forceinline__ void attn_merge_one(const AttnArgs& a, int b, int qh, int nc, int d,
                                               int lane, uint32_t ty, uint32_t* err) {
  constexpr int kBatch = 32;
  const int kvh = qh / G, h = qh % G;
  const size_t stride = (size_t)G * (2 + kHD);
  const uint64_t* w = a.rec + (((size_t)b * a.n_kv + kvh) * a.nchunks * G + h) * (2 + kHD);
  auto fix = [&](uint64_t& v, const uint64_t* p) {     // wait for the record's tag
    long n = 0;
    while ((uint32_t)(v >> 32) != ty && spin_more(n, err)) v = M3_COH_LOAD(p);
  };
  float M = -INFINITY, m0 = -INFINITY;
  if (lane < nc) m0 = M = rec_load(w + (size_t)lane * stride, ty, err);
  for (int c = lane + 64; c < nc; c += 64) M = fmaxf(M, rec_load(w + c * stride, ty, err));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float L = 0.f, A = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const int c = c0 + lane, cn = min(64, nc - c0);
    const uint64_t* wl = w + (size_t)c * stride + 1;
    uint64_t lr = c < nc ? M3_COH_LOAD(wl) : 0;
    uint64_t raw[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      raw[u] = u < cn ? M3_COH_LOAD(w + (size_t)(c0 + u) * stride + 2 + d) : 0;
    float e = 0.f, l = 0.f;
    if (c < nc) {
      const float mv = c0 == 0 ? m0 : rec_load(w + c * stride, ty, err);
      e = exp2f(mv - M);
      fix(lr, wl);
      l = __uint_as_float((uint32_t)lr);
    }
    for (int u0 = 0; u0 < cn; u0 += kBatch) {
      if (u0 > 0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          raw[u] = u0 + u < cn ? M3_COH_LOAD(w + (size_t)(c0 + u0 + u) * stride + 2 + d) : 0;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (u0 + u >= cn) break;
        fix(raw[u], w + (size_t)(c0 + u0 + u) * stride + 2 + d);
        const float eu = __shfl(e, u0 + u), lu = __shfl(l, u0 + u);
        L = fmaf(lu, eu, L);
        A = fmaf(__uint_as_float((uint32_t)raw[u]), eu, A);
      }
    }
  }
  act_store1<true>(a.out, (size_t)b * a.n_q * kHD + (size_t)qh * kHD + d, f2bf(A / L), ty);
}

// The whole attention phase for one workgroup (512 threads).  ebase: the
// launch's epoch base; phase: this phase's index; staged(): called once the
// first items' q are staged (the phase clock).
template <int G, int CH, class Staged>
__device__ __forceinline__ void attn_phase(const AttnArgs& a, uint8_t* smem, int wg, int nwg,
                                           uint32_t ebase, int phase, uint32_t* err,
                                           Staged staged) {
  const uint32_t tq = tag_of(a.pqkv, ebase), ty = tag_of(phase, ebase);
  // the thread index through an opaque copy: what the phase derives from it
  // is computed here, not hoisted out of the frame's phase loop, where it
  // would hold registers through the GEMV phases (which run at the limit)
  int tx = threadIdx.x;
  asm volatile("" : "+v"(tx));
  int pos = a.pos;
  if (a.frame) {
    // a frame past the cache writes the last slot and raises the error
    // word, which ends the launch's waits (the state must be recorded again)
    const long p = (long)a.pos0 + (long)*a.frame;
    pos = p < a.max_pos ? (int)p : a.max_pos - 1;
    if (p >= a.max_pos && wg == 0 && tx == 0) st4<true>(err, 0, M3_ERR_ATTN_FULL);
  }
  const int T = pos + 1, nc = (T + CH - 1) / CH;
  const int nbk = a.B * a.n_kv, items = nbk * nc;
  const int half = tx >> 8, tid = tx & 255, lane = tid & 63, hw = tid >> 6;
  AttnLds<G, CH>& L = reinterpret_cast<AttnLds<G, CH>*>(smem)[half];
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + 2 * sizeof(AttnLds<G, CH>)) + half * (G + 2) * kHD;
  uint16_t* kvs = qs + G * kHD;        // this position's key and value rows
  // item i (chunk-major: the chunks holding pos, which wait for QKV's K and V
  // rows, come last) goes to workgroup (i + nwg / 2) % nwg, half (i / nwg) % 2
  const int me = (wg + nwg / 2) % nwg;
  for (int r0 = 0; r0 < items; r0 += 2 * nwg) {
    const int it = r0 + half * nwg + me;
    const bool live = it < items;
    const int chunk = live ? it / nbk : 0, bk = live ? it % nbk : 0;
    const int b = bk / a.n_kv, kvh = bk % a.n_kv;
    const int t0 = chunk * CH, n = live ? min(T - t0, CH) : 1;
    const bool last = live && chunk == nc - 1;
    const size_t base = ((size_t)b * a.n_kv + kvh) * (size_t)a.max_pos * kHD;
    uint16_t* kb = a.k_cache + base;
    uint16_t* vb = a.v_cache + base;
    AttnRegs<G, CH> R;
    if (live) attn_load_kv(R, kb, vb, t0, n, tid);
    // tasks (one per wave at a time): the G query heads, then for the chunk
    // holding pos its key (normed, rotated) and value (copied) into the cache
    const int ntask = live ? G + (last ? 2 : 0) : 0;
    for (int k = hw; k < ntask; k += 4) {
      const int head = k < G ? kvh * G + k : (k == G ? a.n_q + kvh : a.n_q + a.n_kv + kvh);
      const size_t e = (size_t)b * a.ldqkv + (size_t)head * kHD + lane;
      uint32_t w0 = ld4<true>(a.qkv, e * 4), w1 = ld4<true>(a.qkv, (e + 64) * 4);
      long ns = 0;
      while (((w0 >> 16) != tq || (w1 >> 16) != tq) && spin_more(ns, err)) {
        w0 = ld4<true>(a.qkv, e * 4);
        w1 = ld4<true>(a.qkv, (e + 64) * 4);
      }
      w0 &= 0xffffu;
      w1 &= 0xffffu;
      uint32_t y0 = w0, y1 = w1;
      if (k <= G)
        head_norm_rope(w0, w1, k < G ? a.q_gamma : a.k_gamma, a.eps, a.rope, pos, lane, y0, y1);
      // q to LDS; the key (normed, rotated) and the value to the cache and to LDS
      uint16_t* dst = k < G ? qs + k * kHD : kvs + (k - G) * kHD;
      dst[lane] = (uint16_t)y0;
      dst[lane + 64] = (uint16_t)y1;
      if (k >= G) {
        uint16_t* c = (k == G ? kb : vb) + (size_t)pos * kHD;
        c[lane] = (uint16_t)y0;
        c[lane + 64] = (uint16_t)y1;
      }
    }
    __syncthreads();
    if (r0 == 0) staged();
    if (last) attn_set_kv_at(R, kvs, kvs + kHD, t0, n, tid, pos);
    attn_compute(R, n, a.scale2, tid, L, [&](int h, int d, float A, float Mx, float Ls) {
      if (!live) return;
      if (nc == 1) {
        act_store1<true>(a.out, (size_t)b * a.n_q * kHD + (size_t)(kvh * G + h) * kHD + d,
                         f2bf(A / Ls), ty);
      } else {
        uint64_t* w = a.rec + ((((size_t)b * a.n_kv + kvh) * a.nchunks + chunk) * G + h) * (2 + kHD);
        if (d == 0) {
          rec_store(w, Mx, ty);
          rec_store(w + 1, Ls, ty);
        }
        rec_store(w + 2 + d, A, ty);
      }
    }, qs);
  }
  __syncthreads();            // the last reads of LDS are done before the next phase stages
  if (nc > 1) {
    const int nm = a.B * a.n_q, qq = tx >> 7, d = tx & 127;
    for (int m0 = 4 * (nwg - 1 - wg); m0 < nm; m0 += 4 * nwg) {
      const int mi = m0 + qq;
      if (mi < nm) attn_merge_one<G>(a, mi / a.n_q, mi % a.n_q, nc, d, tx & 63, ty, err);
    }
  }
}

}  // namespace m3
