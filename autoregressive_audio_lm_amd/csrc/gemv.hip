// gemv.hip -- RMSNorm-fused skinny GEMV/GEMM over packed bf16 / int8-row /
// int8-group-128 weights for gfx950 (MI355X).
//
// What is computed (TensorFold PR #987, precision list and "What it adds";
// DiffSynth-Studio MiniMax-Music3 model overview):
//   a = x                              (no norm)
//   a[b,k] = bf16(x[b,k] * r_b * g[k]) r_b = (mean_k x^2 + eps)^-1/2, fp32
//   y[b,n] = epi( sum_k W[n,k] a[b,k] ) with fp32 accumulation.
//
// Design (MI355X-first):
//  * The weights are the only large stream (the decode is bandwidth bound:
//    diffusers issue #14486 item 4 counts ~23 GB of weight reads per frame).
//    They are packed in 1 KB tiles (16 rows x 64 B) so that one 16-byte load
//    per lane of a wave64 fetches a whole tile contiguously.  Every weight
//    byte is read exactly once per call.
//  * A workgroup of 8 waves owns a block of 16 output rows; wave w owns a
//    fixed slice of K (a function of K only).  The reduction order of every
//    output therefore depends only on K -- never on N, B, the grid or where a
//    slice of rows starts -- so a sliced lm_head reproduces the full one bit
//    for bit, and row b never depends on the other rows.
//  * The activation block (after the fused RMSNorm) is staged once per
//    workgroup in LDS (row stride padded by 16 B against bank conflicts) and
//    re-used for every tile; workgroups loop over row blocks when there are
//    more blocks than resident workgroups.
//  * Few rows (B < 8): VALU path, v_dot2_f32_bf16 on bf16 pairs; lane l holds
//    row l%16 and one 16-byte K-chunk of each tile, partial sums meet with two
//    cross-lane exchanges.  B >= 8: the product is a real dense contraction
//    and goes to v_mfma_f32_16x16x32_bf16 (A = 16 activation rows, B = the
//    weight tile, exactly the packed lane layout).
//  * int8 is dequantised to bf16 exactly (|q| <= 127 has 7 significant bits)
//    with one SDWA sign-extending convert per byte; scales are applied per row
//    (i8row) or per group of 128 along K (i8g128).
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBatchTiles = 8;         // weight tiles in flight per wave and batch

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct Params {
  const uint8_t* w;
  int N, K, Kp, T, nblocks;
  size_t bbytes;
  const uint16_t* x;
  int ldx, B;
  const float* gamma;
  float eps;
  int stub_group, stub_voff;
  void* y;
  int ldy, out_f32, epi;
  const uint16_t* res;
  int ldr;
  int lds_rows;        // activation rows staged in LDS (0: direct global reads)
};

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, a), acc, false);
}

// four int8 (one dword) -> two dwords of bf16 pairs (exact)
__device__ __forceinline__ void i8x4_to_bf16x4(uint32_t v, uint32_t& lo, uint32_t& hi) {
  float f0 = (float)(int8_t)(v & 0xffu);
  float f1 = (float)(int8_t)((v >> 8) & 0xffu);
  float f2 = (float)(int8_t)((v >> 16) & 0xffu);
  float f3 = (float)((int32_t)v >> 24);
  lo = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
  hi = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
}

__device__ __forceinline__ void i8x16_to_bf16(const uint4& q, uint32_t* o) {
  i8x4_to_bf16x4(q.x, o[0], o[1]);
  i8x4_to_bf16x4(q.y, o[2], o[3]);
  i8x4_to_bf16x4(q.z, o[4], o[5]);
  i8x4_to_bf16x4(q.w, o[6], o[7]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// source column of operand element k (8-aligned chunk) in x
__device__ __forceinline__ int src_col(const Params& p, int k) {
  if (p.stub_group <= 0) return k;
  return p.stub_voff + (k / (128 * p.stub_group)) * 128 + (k & 127);
}

__device__ __forceinline__ uint4 load_x8(const Params& p, int b, int k) {
  return *reinterpret_cast<const uint4*>(p.x + (size_t)b * p.ldx + src_col(p, k));
}

// Stage the operand rows in LDS (bf16, row stride Kp + 8), fusing the norm.
__device__ void stage_activations(const Params& p, uint16_t* act, float* ss_buf) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int stride = p.Kp + 8;
  const int nchunk = p.Kp >> 3;
  for (int b = 0; b < p.lds_rows; ++b) {
    float ss = 0.f;
    for (int i = tid; i < nchunk; i += kThreads) {
      const int k = i << 3;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k < p.K) v = load_x8(p, b, k);
      *reinterpret_cast<uint4*>(act + (size_t)b * stride + k) = v;
      if (p.gamma) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a0 = bf2f(wv[j] & 0xffffu), a1 = bf2f(wv[j] >> 16);
          ss = fmaf(a0, a0, ss);
          ss = fmaf(a1, a1, ss);
        }
      }
    }
    if (p.gamma) {
      ss = wave_sum(ss);
      if (lane == 0) ss_buf[b * kWaves + wave] = ss;
    }
  }
  __syncthreads();
  if (!p.gamma) return;
  for (int b = 0; b < p.lds_rows; ++b) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += ss_buf[b * kWaves + w];
    const float r = 1.0f / sqrtf(tot / (float)p.K + p.eps);
    for (int i = tid; i < nchunk; i += kThreads) {
      const int k = i << 3;
      if (k >= p.K) continue;
      uint4* ptr = reinterpret_cast<uint4*>(act + (size_t)b * stride + k);
      uint4 v = *ptr;
      const float4 g0 = *reinterpret_cast<const float4*>(p.gamma + k);
      const float4 g1 = *reinterpret_cast<const float4*>(p.gamma + k + 4);
      const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = (bf2f(wv[j] & 0xffffu) * r) * g[2 * j];
        const float a1 = (bf2f(wv[j] >> 16) * r) * g[2 * j + 1];
        wv[j] = f2bf(a0) | (f2bf(a1) << 16);
      }
      *ptr = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  }
  __syncthreads();
}

template <bool LDS>
__device__ __forceinline__ uint4 act8(const Params& p, const uint16_t* act, int b, int k) {
  if constexpr (LDS) {
    return *reinterpret_cast<const uint4*>(act + (size_t)b * (p.Kp + 8) + k);
  } else {
    if (k >= p.K) return make_uint4(0, 0, 0, 0);
    return load_x8(p, b, k);
  }
}

// Epilogue for one output element (or a gate/up pair) after the cross-wave sum.
__device__ __forceinline__ void store_out(const Params& p, int b, int n, float v) {
  if (p.out_f32) {
    reinterpret_cast<float*>(p.y)[(size_t)b * p.ldy + n] = v;
    return;
  }
  uint32_t o = f2bf(v);
  if (p.epi == M3_EPI_RESIDUAL) o = f2bf(bf2f(p.res[(size_t)b * p.ldr + n]) + bf2f(o));
  reinterpret_cast<uint16_t*>(p.y)[(size_t)b * p.ldy + n] = (uint16_t)o;
}

template <int FMT>
__device__ __forceinline__ float row_scale(const uint8_t* blk, const Params& p, int r) {
  if constexpr (FMT == M3_I8ROW)
    return reinterpret_cast<const float*>(blk + (size_t)p.T * kTileBytes)[r];
  return 1.0f;
}

// Cross-wave reduction in fixed wave order, scale, epilogue, store.
template <int FMT, int NB, bool GLU>
__device__ void finish_block(const Params& p, const uint8_t* blk, int rb, const float* red) {
  const int tid = threadIdx.x;
  if constexpr (GLU) {
    for (int t = tid; t < p.B * 8; t += kThreads) {
      const int b = t >> 3, pr = t & 7;
      const int n = rb * 16 + 2 * pr;
      if (n + 1 >= p.N) continue;
      float vg = 0.f, vu = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        vg += red[(w * NB + b) * 16 + 2 * pr];
        vu += red[(w * NB + b) * 16 + 2 * pr + 1];
      }
      vg *= row_scale<FMT>(blk, p, 2 * pr);
      vu *= row_scale<FMT>(blk, p, 2 * pr + 1);
      const float g = bf2f(f2bf(vg)), u = bf2f(f2bf(vu));
      const float s = g / (1.0f + expf(-g));
      reinterpret_cast<uint16_t*>(p.y)[(size_t)b * p.ldy + (n >> 1)] = (uint16_t)f2bf(s * u);
    }
    return;
  }
  for (int t = tid; t < p.B * 16; t += kThreads) {
    const int b = t >> 4, r = t & 15;
    const int n = rb * 16 + r;
    if (n >= p.N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * NB + b) * 16 + r];
    v *= row_scale<FMT>(blk, p, r);
    store_out(p, b, n, v);
  }
}

// ---------------------------------------------------------------------------
// VALU path: NB activation rows (B <= NB), lane = (row l%16, K-chunk l/16).
// ---------------------------------------------------------------------------
template <int FMT, int NB, bool LDS>
__device__ __forceinline__ void valu_tile(const Params& p, const uint16_t* act, const uint4& wv,
                                          int k0, float* acc) {
  const int lane = threadIdx.x & 63, c = lane >> 4;
  if constexpr (FMT == M3_BF16) {
    const int kk = k0 + c * 8;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < p.B) {
        const uint4 av = act8<LDS>(p, act, b, kk);
        float a = acc[b];
        a = dot2(wv.x, av.x, a);
        a = dot2(wv.y, av.y, a);
        a = dot2(wv.z, av.z, a);
        a = dot2(wv.w, av.w, a);
        acc[b] = a;
      }
    }
  } else {
    const int kk = k0 + c * 16;
    uint32_t wb[8];
    i8x16_to_bf16(wv, wb);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < p.B) {
        const uint4 a0 = act8<LDS>(p, act, b, kk);
        const uint4 a1 = act8<LDS>(p, act, b, kk + 8);
        float a = acc[b];
        a = dot2(wb[0], a0.x, a);
        a = dot2(wb[1], a0.y, a);
        a = dot2(wb[2], a0.z, a);
        a = dot2(wb[3], a0.w, a);
        a = dot2(wb[4], a1.x, a);
        a = dot2(wb[5], a1.y, a);
        a = dot2(wb[6], a1.z, a);
        a = dot2(wb[7], a1.w, a);
        acc[b] = a;
      }
    }
  }
}

template <int FMT, int NB, bool LDS, bool GLU>
__device__ void valu_block(const Params& p, const uint16_t* act, float* red, int rb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* blk = p.w + (size_t)rb * p.bbytes;
  const int TK = tile_k(FMT);
  const int tpu = FMT == M3_I8G128 ? 2 : 1;
  const int units = p.T / tpu;
  const int t_lo = (units * wave / kWaves) * tpu;
  const int t_hi = (units * (wave + 1) / kWaves) * tpu;
  const float* gscale = reinterpret_cast<const float*>(blk + (size_t)p.T * kTileBytes);

  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  float gacc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) gacc[b] = 0.f;

  for (int t0 = t_lo; t0 < t_hi; t0 += kBatchTiles) {
    uint4 wv[kBatchTiles];
#pragma unroll
    for (int i = 0; i < kBatchTiles; ++i)
      if (t0 + i < t_hi)
        wv[i] = *reinterpret_cast<const uint4*>(blk + (size_t)(t0 + i) * kTileBytes + lane * 16);
#pragma unroll
    for (int i = 0; i < kBatchTiles; ++i) {
      if (t0 + i < t_hi) {
        const int t = t0 + i;
        if constexpr (FMT == M3_I8G128) {
          valu_tile<FMT, NB, LDS>(p, act, wv[i], t * TK, gacc);
          if (t & 1) {
            const float s = gscale[(t >> 1) * 16 + (lane & 15)];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              acc[b] = fmaf(s, gacc[b], acc[b]);
              gacc[b] = 0.f;
            }
          }
        } else {
          valu_tile<FMT, NB, LDS>(p, act, wv[i], t * TK, acc);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float v = acc[b];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) red[(wave * NB + b) * 16 + lane] = v;
  }
  __syncthreads();
  finish_block<FMT, NB, GLU>(p, blk, rb, red);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// MFMA path: NT tiles of 16 activation rows.  D[i][j] += sum_k A[i][k] B[k][j]
// with A = activations (row i = lane%16 of tile), B = weight tile (column j =
// weight row lane%16); lane l supplies k = 8*(l/16) .. +7 of each operand and
// receives D[4*(l/16) + q][l%16], q = 0..3.
// ---------------------------------------------------------------------------
template <int FMT, int NT, bool LDS>
__device__ __forceinline__ void mfma_tile(const Params& p, const uint16_t* act, const uint4& wv,
                                          int k0, f32x4_t* acc) {
  const int lane = threadIdx.x & 63, c = lane >> 4, i = lane & 15;
  if constexpr (FMT == M3_BF16) {
    const int kk = k0 + c * 8;
    const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wv);
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      const int b = min(bt * 16 + i, p.B - 1);
      const uint4 av = act8<LDS>(p, act, b, kk);
      acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), bw,
                                                        acc[bt], 0, 0, 0);
    }
  } else {
    const int kk = k0 + c * 16;
    uint32_t wb[8];
    i8x16_to_bf16(wv, wb);
    const bf16x8_t blo = __builtin_bit_cast(bf16x8_t, make_uint4(wb[0], wb[1], wb[2], wb[3]));
    const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, make_uint4(wb[4], wb[5], wb[6], wb[7]));
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      const int b = min(bt * 16 + i, p.B - 1);
      const uint4 a0 = act8<LDS>(p, act, b, kk);
      const uint4 a1 = act8<LDS>(p, act, b, kk + 8);
      acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), blo,
                                                        acc[bt], 0, 0, 0);
      acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), bhi,
                                                        acc[bt], 0, 0, 0);
    }
  }
}

template <int FMT, int NT, bool LDS, bool GLU>
__device__ void mfma_block(const Params& p, const uint16_t* act, float* red, int rb) {
  constexpr int NB = NT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* blk = p.w + (size_t)rb * p.bbytes;
  const int TK = tile_k(FMT);
  const int tpu = FMT == M3_I8G128 ? 2 : 1;
  const int units = p.T / tpu;
  const int t_lo = (units * wave / kWaves) * tpu;
  const int t_hi = (units * (wave + 1) / kWaves) * tpu;
  const float* gscale = reinterpret_cast<const float*>(blk + (size_t)p.T * kTileBytes);

  f32x4_t acc[NT], gacc[NT];
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) {
    acc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    gacc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = t_lo; t0 < t_hi; t0 += kBatchTiles) {
    uint4 wv[kBatchTiles];
#pragma unroll
    for (int i = 0; i < kBatchTiles; ++i)
      if (t0 + i < t_hi)
        wv[i] = *reinterpret_cast<const uint4*>(blk + (size_t)(t0 + i) * kTileBytes + lane * 16);
#pragma unroll
    for (int i = 0; i < kBatchTiles; ++i) {
      if (t0 + i < t_hi) {
        const int t = t0 + i;
        if constexpr (FMT == M3_I8G128) {
          mfma_tile<FMT, NT, LDS>(p, act, wv[i], t * TK, gacc);
          if (t & 1) {
            const float s = gscale[(t >> 1) * 16 + (lane & 15)];
#pragma unroll
            for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[bt][q] = fmaf(s, gacc[bt][q], acc[bt][q]);
              gacc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          }
        } else {
          mfma_tile<FMT, NT, LDS>(p, act, wv[i], t * TK, acc);
        }
      }
    }
  }
#pragma unroll
  for (int bt = 0; bt < NT; ++bt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      red[(wave * NB + bt * 16 + 4 * (lane >> 4) + q) * 16 + (lane & 15)] = acc[bt][q];
  __syncthreads();
  finish_block<FMT, NB, GLU>(p, blk, rb, red);
  __syncthreads();
}

// GLU selects the SwiGLU epilogue at compile time (its own kernel symbol, so
// the gate/up GEMVs can be told apart in a profile).
template <int FMT, int NB, bool MFMA, bool LDS, bool GLU>
__global__ __launch_bounds__(kThreads) void gemv_kernel(Params p) {
  extern __shared__ __align__(16) uint8_t smem[];
  float* red = reinterpret_cast<float*>(smem);                       // [kWaves][NB][16]
  float* ss_buf = red + kWaves * NB * 16;                            // [lds_rows][kWaves]
  uint16_t* act = reinterpret_cast<uint16_t*>(ss_buf + M3_MAX_B * kWaves);
  if (LDS) stage_activations(p, act, ss_buf);
  for (int rb = blockIdx.x; rb < p.nblocks; rb += gridDim.x) {
    if constexpr (MFMA)
      mfma_block<FMT, NB / 16, LDS, GLU>(p, act, red, rb);
    else
      valu_block<FMT, NB, LDS, GLU>(p, act, red, rb);
  }
}

template <int FMT, int NB, bool MFMA, bool LDS, bool GLU>
hipError_t configure_one() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemv_kernel<FMT, NB, MFMA, LDS, GLU>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  return status;
}

template <int FMT, int NB, bool MFMA, bool LDS>
hipError_t launch_one(const Params& p, int grid, size_t smem, hipStream_t s) {
  const bool glu = p.epi == M3_EPI_SWIGLU;
  const hipError_t e = glu ? configure_one<FMT, NB, MFMA, LDS, true>()
                           : configure_one<FMT, NB, MFMA, LDS, false>();
  if (e != hipSuccess) return e;
  if (glu)
    hipLaunchKernelGGL((gemv_kernel<FMT, NB, MFMA, LDS, true>), dim3(grid), dim3(kThreads), smem, s, p);
  else
    hipLaunchKernelGGL((gemv_kernel<FMT, NB, MFMA, LDS, false>), dim3(grid), dim3(kThreads), smem, s, p);
  return hipGetLastError();
}

template <int FMT, bool LDS>
hipError_t dispatch_b(const Params& p, int grid, size_t smem, hipStream_t s) {
  const int B = p.B;
  if (B <= 1) return launch_one<FMT, 1, false, LDS>(p, grid, smem, s);
  if (B <= 2) return launch_one<FMT, 2, false, LDS>(p, grid, smem, s);
  if (B <= 4) return launch_one<FMT, 4, false, LDS>(p, grid, smem, s);
  if (B < 8) return launch_one<FMT, 8, false, LDS>(p, grid, smem, s);
  if (B <= 16) return launch_one<FMT, 16, true, LDS>(p, grid, smem, s);
  if (B <= 32) return launch_one<FMT, 32, true, LDS>(p, grid, smem, s);
  if (B <= 48) return launch_one<FMT, 48, true, LDS>(p, grid, smem, s);
  return launch_one<FMT, 64, true, LDS>(p, grid, smem, s);
}

template <int FMT, bool LDS, bool GLU>
hipError_t configure_epi() {
  const hipError_t es[] = {
      configure_one<FMT, 1, false, LDS, GLU>(),  configure_one<FMT, 2, false, LDS, GLU>(),
      configure_one<FMT, 4, false, LDS, GLU>(),  configure_one<FMT, 8, false, LDS, GLU>(),
      configure_one<FMT, 16, true, LDS, GLU>(),  configure_one<FMT, 32, true, LDS, GLU>(),
      configure_one<FMT, 48, true, LDS, GLU>(),  configure_one<FMT, 64, true, LDS, GLU>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

template <int FMT, bool LDS>
hipError_t configure_fmt() {
  const hipError_t es[] = {configure_epi<FMT, LDS, false>(), configure_epi<FMT, LDS, true>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

int nb_of(int B) {
  if (B <= 1) return 1;
  if (B <= 2) return 2;
  if (B <= 4) return 4;
  if (B < 8) return 8;
  return (B + 15) / 16 * 16;
}

size_t fixed_smem(int NB) { return (size_t)kWaves * NB * 16 * 4 + (size_t)M3_MAX_B * kWaves * 4; }

}  // namespace

size_t gemv_smem_bytes(int fmt, int K, int B, bool has_gamma) {
  const size_t fixed = fixed_smem(nb_of(B));
  const size_t act = (size_t)B * (k_pad(fmt, K) + 8) * 2;
  if (has_gamma || fixed + act <= 96 * 1024) return fixed + act;
  return fixed;
}

hipError_t gemv_prepare() {
  const hipError_t es[] = {configure_fmt<M3_BF16, true>(),   configure_fmt<M3_BF16, false>(),
                           configure_fmt<M3_I8ROW, true>(),  configure_fmt<M3_I8ROW, false>(),
                           configure_fmt<M3_I8G128, true>(), configure_fmt<M3_I8G128, false>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_gemv(const GemvDesc& d, hipStream_t s) {
  Params p;
  p.w = static_cast<const uint8_t*>(d.w);
  p.N = d.N;
  p.K = d.K;
  p.Kp = k_pad(d.fmt, d.K);
  p.T = n_tiles(d.fmt, d.K);
  p.nblocks = n_blocks(d.N);
  p.bbytes = block_bytes(d.fmt, d.K);
  p.x = d.x;
  p.ldx = d.ldx;
  p.B = d.B;
  p.gamma = d.gamma;
  p.eps = d.eps;
  p.stub_group = d.stub_group;
  p.stub_voff = d.stub_voff;
  p.y = d.y;
  p.ldy = d.ldy;
  p.out_f32 = d.out_f32;
  p.epi = d.epi;
  p.res = d.res;
  p.ldr = d.ldr;
  const size_t fixed = fixed_smem(nb_of(d.B));
  const size_t smem = gemv_smem_bytes(d.fmt, d.K, d.B, d.gamma != nullptr);
  const bool lds = smem > fixed;
  p.lds_rows = lds ? d.B : 0;
  // resident workgroups per CU from LDS (8 waves each, at most 2 per CU)
  int per_cu = (int)((160 * 1024) / (smem + 1024));
  per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
  int grid = 256 * per_cu;
  if (grid > p.nblocks) grid = p.nblocks;
  switch (d.fmt) {
    case M3_BF16:
      return lds ? dispatch_b<M3_BF16, true>(p, grid, smem, s)
                 : dispatch_b<M3_BF16, false>(p, grid, smem, s);
    case M3_I8ROW:
      return lds ? dispatch_b<M3_I8ROW, true>(p, grid, smem, s)
                 : dispatch_b<M3_I8ROW, false>(p, grid, smem, s);
    default:
      return lds ? dispatch_b<M3_I8G128, true>(p, grid, smem, s)
                 : dispatch_b<M3_I8G128, false>(p, grid, smem, s);
  }
}

}  // namespace m3
