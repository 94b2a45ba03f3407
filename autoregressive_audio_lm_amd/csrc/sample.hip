// sample.hip -- Philox-4x32-10 Gumbel-argmax over [B, V] logits.
//
// Gumbel-argmax draws exactly from softmax(l/T) (diffusers issue #14486,
// item 3, where it replaces softmax + multinomial).  The noise of vocab id i
// in batch row b of draw d of frame f is a pure function of
// (seed, i, b, f, d): Philox-4x32-10 (Salmon et al., "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC'11) keyed by the seed with counter (i>>2, b, f, d),
// word i&3 (the Philox counters of TensorFold PR #987's draw).  Noise keyed by
// the absolute id makes a vocab slice draw the same id as the full, masked
// vocabulary.  Every floating-point step is one IEEE fp32 operation in a
// fixed order (no contraction), so the draw is bit-reproducible.
//
// Two small kernels: per (row, chunk of 1024 ids) a workgroup finds its best
// (z, index); one wave per row then reduces the chunk winners.  The order
// (z descending with NaN on top, then index ascending) is total, so the
// result does not depend on how the reduction is arranged.
#include "cfg_impl.h"

#include <mutex>

#pragma clang fp contract(off)

namespace m3 {
namespace {

constexpr int kChunk = 1024;
constexpr int kSThreads = 256;

__global__ __launch_bounds__(kSThreads) void gumbel_partial(SampleDesc d) {
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t frame = d.frame_dev ? *d.frame_dev : d.frame;
  const float invT = inv_temperature(d.temperature);
  const uint32_t k0 = (uint32_t)d.seed, k1 = (uint32_t)(d.seed >> 32);
  float bz = -INFINITY;
  int bj = 0x7fffffff;
  uint32_t cached = 0xffffffffu;
  uint32_t words[4] = {0, 0, 0, 0};
  const int j0 = chunk * kChunk + tid * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = j0 + e;
    if (j >= d.V) break;
    const int32_t id = d.ids ? d.ids[j] : d.index_base + j;
    float z;
    if (d.valid_lo < d.valid_hi && (id < d.valid_lo || id >= d.valid_hi)) {
      z = -INFINITY;
    } else {
      float g;
      if (d.noise) {
        g = d.noise[(size_t)b * d.V + j];
      } else {
        const uint32_t grp = (uint32_t)id >> 2;
        if (grp != cached) {
          words[0] = grp;
          words[1] = (uint32_t)b;
          words[2] = frame;
          words[3] = d.draw;
          philox10(words, k0, k1);
          cached = grp;
        }
        g = gumbel_from_word(words[(uint32_t)id & 3u]);
      }
      z = gumbel_z(d.logits[(size_t)b * d.ldl + j], invT, g);
    }
    if (above(z, j, bz, bj)) {
      bz = z;
      bj = j;
    }
  }
  best_reduce(bz, bj, 64);
  __shared__ Best sb[kSThreads / 64];
  if (lane == 0) sb[wave] = Best{bz, bj};
  __syncthreads();
  if (tid == 0) {
    Best r = sb[0];
    for (int w = 1; w < kSThreads / 64; ++w)
      if (above(sb[w].z, sb[w].j, r.z, r.j)) r = sb[w];
    reinterpret_cast<Best*>(d.ws)[(size_t)b * gridDim.x + chunk] = r;
  }
}

__global__ __launch_bounds__(64) void gumbel_final(SampleDesc d, int nchunk) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const Best* part = reinterpret_cast<const Best*>(d.ws) + (size_t)b * nchunk;
  float bz = -INFINITY;
  int bj = 0x7fffffff;
  for (int c = lane; c < nchunk; c += 64) {
    const Best r = part[c];
    if (above(r.z, r.j, bz, bj)) {
      bz = r.z;
      bj = r.j;
    }
  }
  best_reduce(bz, bj, 64);
  if (lane == 0) {
    // an all -inf row keeps every element tied at -inf: the lowest index wins
    const int j = bj;
    d.out[(size_t)b * d.out_stride] = d.ids ? d.ids[j] : d.index_base + j;
  }
}

// ---- the reference's draw: guidance over row pairs, top-k, Gumbel-argmax ------
// One workgroup of 1024 threads per song; the draw itself is cfg_song
// (cfg_impl.h), which the persistent frame runs too.
constexpr int kCfgThreads = 1024;

template <int E>
__global__ __launch_bounds__(kCfgThreads) void cfg_topk_kernel(CfgDesc d) {
  __shared__ CfgShared<kCfgThreads> sh;
  cfg_song<E, kCfgThreads, false>(d, blockIdx.x, threadIdx.x, sh, kPlain);
}

template <int E>
hipError_t launch_cfg_e(const CfgDesc& d, hipStream_t s) {
  hipLaunchKernelGGL(cfg_topk_kernel<E>, dim3(d.S), dim3(kCfgThreads), 0, s, d);
  return hipGetLastError();
}

}  // namespace

size_t sample_ws_bytes(int B, int V) {
  const size_t nchunk = ((size_t)V + kChunk - 1) / kChunk;
  return (size_t)B * nchunk * sizeof(Best);
}

hipError_t launch_cfg_draw(const CfgDesc& d, hipStream_t s) {
  if (d.V < 1 || d.V > kCfgMaxV || d.S < 1 || d.top_k < 1) return hipErrorInvalidValue;
  const int e = (d.V + kCfgThreads - 1) / kCfgThreads;
  if (e <= 1) return launch_cfg_e<1>(d, s);
  if (e <= 2) return launch_cfg_e<2>(d, s);
  if (e <= 4) return launch_cfg_e<4>(d, s);
  if (e <= 8) return launch_cfg_e<8>(d, s);
  if (e <= 16) return launch_cfg_e<16>(d, s);
  return launch_cfg_e<32>(d, s);
}

// ---- the allocation-free draw's scratch ------------------------------------------
// One fixed array per device for the per-chunk winners of
// m3_gumbel_argmax_noalloc (callers that cannot allocate).  In host code the
// array's name is only a stand-in: its device address is looked up once per
// device, with that device current, and that address is what kernels get.
static __device__ __align__(256) uint8_t scratch[kSampleScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t sample_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_sample(const SampleDesc& d, hipStream_t s) {
  const int nchunk = (d.V + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(gumbel_partial, dim3(nchunk, d.B), dim3(kSThreads), 0, s, d);
  hipLaunchKernelGGL(gumbel_final, dim3(d.B), dim3(64), 0, s, d, nchunk);
  return hipGetLastError();
}

}  // namespace m3
