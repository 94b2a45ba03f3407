// frame.hip -- the small per-frame kernels around the GEMVs: depth-decoder
// input embedding, frame-embedding feedback with the GPU-side frame counter
// and 16-frame code ring, and state initialisation.
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

// d[b, :] = bf16(u[b, :] + E[c, :]), c = codes[b*8 + col] - base (0 if out of range)
__global__ __launch_bounds__(256) void depth_input_kernel(const uint16_t* u, const uint16_t* E,
                                                          const int32_t* codes, int col,
                                                          int32_t base, int n_codes, int B,
                                                          int D, uint16_t* out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;   // one thread per 8 elements
  const int per_row = D >> 3;
  if (idx >= (long)B * per_row) return;
  const int b = (int)(idx / per_row), k = (int)(idx % per_row) * 8;
  int c = codes[b * 8 + col] - base;
  if (c < 0 || c >= n_codes) c = 0;
  const uint4 uv = *reinterpret_cast<const uint4*>(u + (size_t)b * D + k);
  const uint4 ev = *reinterpret_cast<const uint4*>(E + (size_t)c * D + k);
  const uint32_t a[4] = {uv.x, uv.y, uv.z, uv.w}, e[4] = {ev.x, ev.y, ev.z, ev.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = f2bf(bf2f(a[j] & 0xffffu) + bf2f(e[j] & 0xffffu));
    const uint32_t hi = f2bf(bf2f(a[j] >> 16) + bf2f(e[j] >> 16));
    o[j] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(out + (size_t)b * D + k) = make_uint4(o[0], o[1], o[2], o[3]);
}

struct FeedbackArgs {
  const uint16_t* tok;           // [n_slice, H]
  const uint16_t* aemb[8];       // [code_vocab, H] for codebooks 1..n_cb-1
  const int32_t* codes;          // [B, 8]
  int32_t vocab_base;
  int n_slice, code_vocab, n_cb, B, H;
  uint16_t* x;
  int32_t* ring;                 // [16, B, 8]
  uint32_t* frame;
};

__global__ __launch_bounds__(256) void feedback_kernel(FeedbackArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = a.H >> 3;
  if (idx < (long)a.B * per_row) {
    const int b = (int)(idx / per_row), k = (int)(idx % per_row) * 8;
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
      int c = a.codes[b * 8 + cb];
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
  if (blockIdx.x == 0) {
    // ring slot of this frame, then advance the counter (only block 0 reads it)
    const uint32_t f = *a.frame;
    for (int i = threadIdx.x; i < a.B * 8; i += 256)
      a.ring[(size_t)(f & 15u) * a.B * 8 + i] = a.codes[i];
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

hipError_t launch_depth_input(const uint16_t* u, const uint16_t* emb, const int32_t* codes,
                              int code_col, int32_t code_base, int n_codes, int B, int D,
                              uint16_t* out, hipStream_t s) {
  const long n = (long)B * (D / 8);
  hipLaunchKernelGGL(depth_input_kernel, dim3((int)((n + 255) / 256)), dim3(256), 0, s, u, emb,
                     codes, code_col, code_base, n_codes, B, D, out);
  return hipGetLastError();
}

hipError_t launch_feedback(const uint16_t* tok_emb_audio, const uint16_t* const* audio_emb,
                           const int32_t* codes, int32_t vocab_base, int n_slice,
                           int code_vocab, int n_cb, int B, int H, uint16_t* x_out, int32_t* ring,
                           uint32_t* frame, hipStream_t s) {
  FeedbackArgs a;
  a.code_vocab = code_vocab;
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
  const long n = (long)B * (H / 8);
  hipLaunchKernelGGL(feedback_kernel, dim3((int)((n + 255) / 256)), dim3(256), 0, s, a);
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
