// m3_sampling.h -- Gumbel noise and the argmax order, shared by the sampler
// kernels and the sampling epilogue of the lm_head/head GEMVs.
//
// Noise of absolute vocab id i, batch row b, frame f, draw d: Philox-4x32-10
// (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) keyed
// by the 64-bit seed with counter (i >> 2, b, f, d); word i & 3; uniform
// u = (2 (w >> 9) + 1) 2^-24 (exact in fp32, inside (0, 1)); G = -log(-log u)
// with a log built from IEEE fp32 operations in a fixed order.  Gumbel-argmax
// draws from softmax(l/T) (diffusers issue #14486, item 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

struct Best {
  float z;
  int j;
};

__device__ __forceinline__ void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// ln x for positive normal x: x = m 2^e with m in (1/sqrt2, sqrt2],
// ln x = e ln2 + 2 atanh((m-1)/(m+1)), atanh t = t + t^3/3 + ... + t^11/11.
__device__ __forceinline__ float log_fixed(float x) {
#pragma clang fp contract(off)
  const uint32_t u = __float_as_uint(x);
  int e = (int)((u >> 23) & 0xffu) - 127;
  float m = __uint_as_float((u & 0x007fffffu) | 0x3f800000u);
  if (m > (float)1.41421356237309504880) {
    m = m * 0.5f;
    e = e + 1;
  }
  const float f = m - 1.0f;
  const float d = m + 1.0f;
  const float t = f / d;
  const float s = t * t;
  float p = 1.0f / 11.0f;
  p = __builtin_fmaf(p, s, 1.0f / 9.0f);
  p = __builtin_fmaf(p, s, 1.0f / 7.0f);
  p = __builtin_fmaf(p, s, 1.0f / 5.0f);
  p = __builtin_fmaf(p, s, 1.0f / 3.0f);
  const float sp = s * p;
  const float r = sp * t;
  float lm = t + r;
  lm = lm + lm;
  const float ef = (float)e;
  constexpr float kLn2Hi = 0x1.62e4p-1f;
  constexpr float kLn2Lo = (float)(0.69314718055994530942 - 0.693145751953125);
  float res = __builtin_fmaf(ef, kLn2Lo, lm);
  res = __builtin_fmaf(ef, kLn2Hi, res);
  return res;
}

__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
#pragma clang fp contract(off)
  const float uu = (float)(((w >> 9) << 1) | 1u) * 0x1p-24f;
  const float l1 = log_fixed(uu);
  const float l2 = log_fixed(-l1);
  return -l2;
}

// z = fl32(l * fl32(1/T)) + g: two roundings, never fused
__device__ __forceinline__ float gumbel_z(float logit, float inv_t, float g) {
#pragma clang fp contract(off)
  const float lt = logit * inv_t;
  return lt + g;
}

__device__ __forceinline__ float inv_temperature(float t) {
#pragma clang fp contract(off)
  return 1.0f / t;
}

// Gumbel noise of one absolute id (a full Philox call)
__device__ __forceinline__ float gumbel_noise(uint64_t seed, uint32_t row, uint32_t frame,
                                              uint32_t draw, uint32_t id) {
  uint32_t c[4] = {id >> 2, row, frame, draw};
  philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return gumbel_from_word(c[id & 3u]);
}

// total order of the argmax: NaN above every number, then value, then the
// lower index.  True if (za, ia) ranks above (zb, ib).
__device__ __forceinline__ bool above(float za, int ia, float zb, int ib) {
  const bool an = za != za, bn = zb != zb;
  if (an != bn) return an;
  if (!an && za != zb) return za > zb;
  return ia < ib;
}

// The best (z, j) over groups of `width` lanes (16 or 64), left in every
// lane of the group.  The order is total, so any pairing gives the same
// winner: DPP quad exchanges and half-row / row mirrors inside a row of 16
// lanes, then (width 64) the permlane swaps between rows.  Every lane of the
// wave must be active.
template <int CTRL>
__device__ __forceinline__ void best_dpp(float& z, int& j) {
  const float oz = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), CTRL, 0xF, 0xF, false));
  const int oj = __builtin_amdgcn_update_dpp(0, j, CTRL, 0xF, 0xF, false);
  if (above(oz, oj, z, j)) {
    z = oz;
    j = oj;
  }
}

__device__ __forceinline__ void best_swap(float& z, int& j, bool rows32) {
  // the swap of a register with itself returns the two partners' values in
  // r[0] / r[1]; this lane's partner is whichever is not its own
  const auto rz = rows32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false)
                         : __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  const auto rj = rows32 ? __builtin_amdgcn_permlane32_swap((uint32_t)j, (uint32_t)j, false, false)
                         : __builtin_amdgcn_permlane16_swap((uint32_t)j, (uint32_t)j, false, false);
  const int lane = threadIdx.x & 63;
  const bool low = rows32 ? lane < 32 : (lane & 16) == 0;
  const float oz = __uint_as_float(low ? rz[1] : rz[0]);
  const int oj = (int)(low ? rj[1] : rj[0]);
  if (above(oz, oj, z, j)) {
    z = oz;
    j = oj;
  }
}

__device__ __forceinline__ void best_reduce(float& z, int& j, int width) {
  best_dpp<0xB1>(z, j);
  best_dpp<0x4E>(z, j);
  best_dpp<0x141>(z, j);
  best_dpp<0x140>(z, j);
  if (width > 16) {
    best_swap(z, j, false);
    best_swap(z, j, true);
  }
}

}  // namespace m3
