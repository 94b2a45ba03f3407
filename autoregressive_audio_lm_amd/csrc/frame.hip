// frame.hip -- the small per-frame kernels around the GEMVs: the last draw
// and the frame-embedding feedback with the GPU-side frame counter and the
// 16-frame code ring, and state initialisation.
//
// DiffSynth-Studio MiniMax-Music3 article, stage 2: after the semantic code,
// the RVQ depth decoder draws the remaining 7 codes one codebook at a time;
// the frame's 8 codes are embedded (embed_tokens of the semantic id plus the
// RVQ audio embeddings of the 7 residual codes), scaled by 8^-1/2 and fed back
// as the next frame's input.  TensorFold PR #987: position and count advance
// on the GPU; the host reads the drawn tokens every 16 frames.
#include "m3_internal.h"

namespace m3 {
namespace {

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

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
};

// the last codebook's draw for row b (same total order as the sampler)
__device__ int last_code(const FeedbackArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  float bz = -INFINITY;
  int bj = 0x7fffffff;
  for (int c = lane; c < a.last_nparts; c += 64) {
    const Best r = a.last_part[(size_t)b * a.last_nparts + c];
    if (above(r.z, r.j, bz, bj)) {
      bz = r.z;
      bj = r.j;
    }
  }
  best_reduce(bz, bj, 64);
  return __shfl(bj, 0, 64);
}

// grid (H / 2048 blocks of 256 threads x 8 values, B).  Block (x, b) handles
// row b; block (0, 0) also writes the last codes, the ring slot and bumps the
// frame counter (it is the only reader of the counter in this kernel).
__global__ __launch_bounds__(256) void feedback_kernel(FeedbackArgs a) {
  __shared__ int c_last[M3_MAX_B_FRAME];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bsel = blockIdx.y;
  const bool leader = blockIdx.x == 0 && blockIdx.y == 0;
  // every block needs its own row's last code; the leader needs all of them
  if (leader) {
    for (int b = wave; b < a.B; b += 4) {
      const int c = last_code(a, b);
      if (lane == 0) c_last[b] = c;
    }
  } else if (wave == 0) {
    const int c = last_code(a, bsel);
    if (lane == 0) c_last[bsel] = c;
  }
  __syncthreads();
  {
    const int b = bsel, k = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (k < a.H) {
    int c0 = a.codes[b * 8] - a.vocab_base;
    if (c0 < 0 || c0 >= a.n_slice) c0 = 0;
    float acc[8];
    const uint4 t = *reinterpret_cast<const uint4*>(a.tok + (size_t)c0 * a.H + k);
    const uint32_t tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = bf2f(tv[j] & 0xffffu);
      acc[2 * j + 1] = bf2f(tv[j] >> 16);
    }
    for (int cb = 1; cb < a.n_cb; ++cb) {
      int c = cb == a.n_cb - 1 ? c_last[b] : a.codes[b * 8 + cb];
      if (c < 0 || c >= a.code_vocab) c = 0;
      const uint4 v = *reinterpret_cast<const uint4*>(a.aemb[cb - 1] + (size_t)c * a.H + k);
      const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf2f(vv[j] & 0xffffu);
        acc[2 * j + 1] += bf2f(vv[j] >> 16);
      }
    }
    const float sc = 1.0f / sqrtf((float)a.n_cb);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f2bf(acc[2 * j] * sc) | (f2bf(acc[2 * j + 1] * sc) << 16);
    *reinterpret_cast<uint4*>(a.x + (size_t)b * a.H + k) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if (leader) {
    const uint32_t f = *a.frame;
    for (int i = threadIdx.x; i < a.B * 8; i += 256) {
      const int b = i >> 3, cb = i & 7;
      const int32_t v = cb == a.n_cb - 1 ? c_last[b] : a.codes[i];
      if (cb == a.n_cb - 1) a.codes[i] = v;
      a.ring[(size_t)(f & 15u) * a.B * 8 + i] = v;
    }
    __syncthreads();
    if (threadIdx.x == 0) *a.frame = f + 1u;
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const uint16_t* src, uint16_t* dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void fill_kernel(uint32_t* dst, uint32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = v;
}

}  // namespace

hipError_t launch_feedback(const uint16_t* tok_emb_audio, const uint16_t* const* audio_emb,
                           int32_t* codes, const Best* last_part, int last_nparts,
                           int32_t vocab_base, int n_slice, int code_vocab, int n_cb, int B,
                           int H, uint16_t* x_out, int32_t* ring, uint32_t* frame, hipStream_t s) {
  FeedbackArgs a;
  a.code_vocab = code_vocab;
  a.last_part = last_part;
  a.last_nparts = last_nparts;
  a.tok = tok_emb_audio;
  for (int i = 0; i < 8; ++i) a.aemb[i] = (i < n_cb - 1) ? audio_emb[i] : nullptr;
  a.codes = codes;
  a.vocab_base = vocab_base;
  a.n_slice = n_slice;
  a.n_cb = n_cb;
  a.B = B;
  a.H = H;
  a.x = x_out;
  a.ring = ring;
  a.frame = frame;
  hipLaunchKernelGGL(feedback_kernel, dim3((H + 2047) / 2048, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_copy_bf16(const uint16_t* src, uint16_t* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* dst, uint32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, v, n);
  return hipGetLastError();
}

}  // namespace m3
