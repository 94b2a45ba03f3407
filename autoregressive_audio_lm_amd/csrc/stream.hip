// stream.hip -- a plain streaming read: the read rate the decode GEMVs are
// held against on this device.
//
// Every workgroup reads 16 bytes per lane per load, the way the GEMVs read
// their weight tiles (raw buffer loads, non-temporal or default cache
// policy), eight loads in flight per lane, over a grid of workgroups that
// walk the buffer in 8 KB strides (loads past the end return zeros); each workgroup folds what it read into one
// word, written to sink[blockIdx.x], so that nothing is optimised away.
#include "m3_internal.h"

namespace m3 {
namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
constexpr int kSThreads = 512;
constexpr int kSUnroll = 8;

template <int AUX>
__global__ __launch_bounds__(kSThreads) void stream_read_kernel(const uint8_t* buf, uint32_t bytes,
                                                                uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0, (int)bytes, 0x00020000);
  const uint32_t step = (uint32_t)gridDim.x * kSThreads * 16u;
  uint32_t acc = 0;
  for (uint32_t base = (uint32_t)blockIdx.x * kSThreads * 16u; base < bytes; base += step * kSUnroll) {
    uint32_t v[kSUnroll];
#pragma unroll
    for (int u = 0; u < kSUnroll; ++u) {
      // past the end: an out-of-range buffer load returns zeros
      // the whole offset goes in the VGPR, the one the range check applies to
      const u32x4v t = __builtin_amdgcn_raw_buffer_load_b128(r, base + u * step + threadIdx.x * 16u, 0, AUX);
      v[u] = t[0] ^ t[1] ^ t[2] ^ t[3];
    }
#pragma unroll
    for (int u = 0; u < kSUnroll; ++u) acc ^= v[u];
  }
  __shared__ uint32_t fold;
  if (threadIdx.x == 0) fold = 0;
  __syncthreads();
  atomicOr(&fold, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = fold;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                              int nontemporal, hipStream_t s) {
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<2>, dim3(workgroups), dim3(kSThreads), 0, s, b,
                       (uint32_t)bytes, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<0>, dim3(workgroups), dim3(kSThreads), 0, s, b,
                       (uint32_t)bytes, sink);
  return hipGetLastError();
}

}  // namespace m3
