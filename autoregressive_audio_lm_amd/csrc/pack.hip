// pack.hip -- load-time quantise + pack into the tiled layout of m3.h.
//
// fp8 (OCP E4M3) weight-only with one scale per row as a further format:
// scale = absmax/448, codes nearest with ties to even (see qf8).
//
// int8 weight-only quantisation on the GPU at load (TensorFold PR #987,
// precision list: a scale per row for the body and lm_head, per group of 128
// for the depth decoder): scale = absmax/127 (one IEEE fp32 division), q =
// nearest integer of W/scale with ties to even, clamped to [-127, 127]; the
// quotient is formed in float64, whose rounding can never move it across a
// half-integer for bf16 numerators and fp32 scales, so q is the correctly
// rounded value.  Gate/up rows can be interleaved in pairs so one GEMV writes
// the SwiGLU of each pair.
#include "m3_internal.h"

namespace m3 {
namespace {

struct PackParams {
  const uint16_t* W;
  int N, K, T, nblocks, flags;
  size_t bbytes;
  uint8_t* out;
};

__device__ __forceinline__ int src_row(const PackParams& p, int n) {
  if (!(p.flags & M3_PACK_GLU_INTERLEAVE)) return n;
  const int F = p.N >> 1;
  return (n & 1) ? F + (n >> 1) : (n >> 1);
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// One wave per (padded row, group): absmax -> scale.  group size = gsz.
template <int FMT>
__global__ __launch_bounds__(256) void scale_kernel(PackParams p) {
  const int lane = threadIdx.x & 63;
  const int G = FMT == M3_I8G128 ? p.K / 128 : 1;
  const int gsz = FMT == M3_I8G128 ? 128 : p.K;
  const float qmax = FMT == M3_FP8ROW ? 448.0f : 127.0f;   // largest code value
  const long task = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long ntask = (long)p.nblocks * 16 * G;
  if (task >= ntask) return;
  const int n = (int)(task / G), g = (int)(task % G);
  float amax = 0.f;
  if (n < p.N) {
    const uint16_t* row = p.W + (size_t)src_row(p, n) * p.K + (size_t)g * gsz;
    for (int k = lane; k < gsz; k += 64) amax = fmaxf(amax, fabsf(bf2f(row[k])));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) {
    const float s = __fdiv_rn(amax, qmax);
    const int rb = n >> 4, r = n & 15;
    float* sc = reinterpret_cast<float*>(p.out + (size_t)rb * p.bbytes + (size_t)p.T * kTileBytes);
    sc[FMT == M3_I8G128 ? r * G + g : r] = s;
  }
}

__device__ __forceinline__ uint32_t q8(float w, float s) {
  if (s == 0.0f) return 0u;
  double t = rint((double)w / (double)s);
  t = t > 127.0 ? 127.0 : (t < -127.0 ? -127.0 : t);
  return (uint32_t)((int)t & 0xff);
}

// fp8 weight-only: the OCP FP8 E4M3 code nearest to w/s (ties to the even
// mantissa), saturated to +-448 (the format has no infinity).  E4M3: sign,
// 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds m * 2^-9.
// The quotient is formed in float64 (as for int8, its rounding cannot move
// it across a midpoint between two codes).
__device__ __forceinline__ uint32_t qf8(float w, float s) {
  if (s == 0.0f) return 0u;
  const double t = (double)w / (double)s;
  if (t != t) return 0x7Fu;                                  // NaN code
  const uint32_t sign = t < 0.0 || (t == 0.0 && signbit(t)) ? 0x80u : 0u;
  const double a = fabs(t);
  if (!(a < 448.0)) return sign | 0x7Eu;
  if (a < 0.015625) return sign | (uint32_t)rint(a * 512.0);   // below 2^-6: steps of 2^-9
  int ex = ilogb(a);                                         // a in [2^ex, 2^(ex+1))
  double mant = rint(scalbn(a, 3 - ex)) - 8.0;               // 3 fraction bits, ties to even
  if (mant >= 8.0) {
    mant = 0.0;
    ++ex;
  }
  if (ex + 7 > 15 || (ex + 7 == 15 && mant >= 7.0)) return sign | 0x7Eu;
  return sign | (uint32_t)((ex + 7) << 3) | (uint32_t)mant;
}

// One thread per 16 packed bytes: (block, tile, lane).
template <int FMT>
__global__ __launch_bounds__(256) void pack_kernel(PackParams p) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)p.nblocks * p.T * 64;
  if (idx >= total) return;
  const int l = (int)(idx & 63);
  const long bt = idx >> 6;
  const int t = (int)(bt % p.T), rb = (int)(bt / p.T);
  const int n = rb * 16 + (l & 15);
  uint8_t* blk = p.out + (size_t)rb * p.bbytes;
  uint4 v = make_uint4(0, 0, 0, 0);
  if constexpr (FMT == M3_BF16) {
    const int k = t * 32 + (l >> 4) * 8;
    if (n < p.N && k < p.K)
      v = *reinterpret_cast<const uint4*>(p.W + (size_t)src_row(p, n) * p.K + k);
  } else {
    const int k = t * 64 + (l >> 4) * 16;
    if (n < p.N && k < p.K) {
      const float* sc = reinterpret_cast<const float*>(blk + (size_t)p.T * kTileBytes);
      const float s = FMT == M3_I8G128 ? sc[(l & 15) * (p.K / 128) + k / 128] : sc[l & 15];
      const uint16_t* src = p.W + (size_t)src_row(p, n) * p.K + k;
      const uint4 a = *reinterpret_cast<const uint4*>(src);
      const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
      const uint32_t h[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float wl = bf2f(h[j] & 0xffffu), wh = bf2f(h[j] >> 16);
        const uint32_t lo = FMT == M3_FP8ROW ? qf8(wl, s) : q8(wl, s);
        const uint32_t hi = FMT == M3_FP8ROW ? qf8(wh, s) : q8(wh, s);
        o[j >> 1] |= (lo | (hi << 8)) << (16 * (j & 1));
      }
      v = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  *reinterpret_cast<uint4*>(blk + (size_t)t * kTileBytes + l * 16) = v;
}

// zero the padding after the scales of each block (i8row, fp8-row: 64 B; g128: rounding)
__global__ __launch_bounds__(256) void pad_kernel(uint8_t* out, int nblocks, size_t bbytes,
                                                  size_t used, size_t pad) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long per = (long)(pad / 4);
  if (idx >= (long)nblocks * per) return;
  const long rb = idx / per, i = idx % per;
  reinterpret_cast<uint32_t*>(out + (size_t)rb * bbytes + used)[i] = 0u;
}

}  // namespace

hipError_t launch_pack(int fmt, const uint16_t* W, int N, int K, int flags, void* packed,
                       hipStream_t s) {
  PackParams p;
  p.W = W;
  p.N = N;
  p.K = K;
  p.T = n_tiles(fmt, K);
  p.nblocks = n_blocks(N);
  p.flags = flags;
  p.bbytes = block_bytes(fmt, K);
  p.out = static_cast<uint8_t*>(packed);
  const long total = (long)p.nblocks * p.T * 64;
  const int grid = (int)((total + 255) / 256);
  if (fmt == M3_BF16) {
    hipLaunchKernelGGL(pack_kernel<M3_BF16>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const int G = fmt == M3_I8G128 ? K / 128 : 1;
  const size_t used = (size_t)p.T * kTileBytes + (size_t)G * 64;
  const size_t pad = p.bbytes - used;
  if (pad > 0) {
    const long n = (long)p.nblocks * (long)(pad / 4);
    hipLaunchKernelGGL(pad_kernel, dim3((int)((n + 255) / 256)), dim3(256), 0, s, p.out,
                       p.nblocks, p.bbytes, used, pad);
  }
  const long ntask = (long)p.nblocks * 16 * G;
  const int sgrid = (int)((ntask + 3) / 4);
  if (fmt == M3_I8ROW) {
    hipLaunchKernelGGL(scale_kernel<M3_I8ROW>, dim3(sgrid), dim3(256), 0, s, p);
    hipLaunchKernelGGL(pack_kernel<M3_I8ROW>, dim3(grid), dim3(256), 0, s, p);
  } else if (fmt == M3_FP8ROW) {
    hipLaunchKernelGGL(scale_kernel<M3_FP8ROW>, dim3(sgrid), dim3(256), 0, s, p);
    hipLaunchKernelGGL(pack_kernel<M3_FP8ROW>, dim3(grid), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(scale_kernel<M3_I8G128>, dim3(sgrid), dim3(256), 0, s, p);
    hipLaunchKernelGGL(pack_kernel<M3_I8G128>, dim3(grid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace m3
