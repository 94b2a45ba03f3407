// frame.hip -- the small per-frame kernels around the GEMVs of the
// graph-replayed frame (the frame end: last draw, feedback, code ring, frame
// counter; see frame_impl.h) and state initialisation.
#include "frame_impl.h"

namespace m3 {
namespace {

// one workgroup of 256 threads per batch row
__global__ __launch_bounds__(256) void feedback_kernel(FeedbackArgs a) {
  __shared__ int c_last[M3_MAX_B_FRAME];
  feedback_run<false>(a, blockIdx.x, gridDim.x, c_last, 0u);
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
                           int H, uint16_t* x_out, int32_t* ring, uint32_t* frame,
                           int32_t end_id, uint32_t* stop, hipStream_t s) {
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
  a.last_part_prod = -1;
  a.th = nullptr;
  a.th_prod = -1;
  a.h_out = nullptr;
  a.seq = nullptr;
  a.end_id = end_id;
  a.stop = stop;
  hipLaunchKernelGGL(feedback_kernel, dim3(B), dim3(256), 0, s, a);
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
