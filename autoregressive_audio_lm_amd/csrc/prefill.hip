// prefill.hip -- prompt prefill: RMSNorm over many rows, and the dense GEMM
// Y[M, N] = A[M, K] . W^T on the matrix cores.
//
// A prompt of about 300 tokens for each of the two CFG rows is 600 rows
// through every body matrix at once ("MiniMax Music 3, local": a prompt of
// 300 tokens per CFG row; TensorFold PR #987: 300 tokens a CFG row), a real
// dense contraction: at 600 rows a bf16 weight byte meets 600 multiply-adds,
// above the matrix cores' ridge, so the bound is the MFMA rate, not HBM.
//
// GEMM.  A workgroup of 4 waves computes a 128 x 128 tile of Y; wave w holds
// rows 64 (w & 1) .. +63 and columns 64 (w >> 1) .. +63 as 4 x 4
// accumulators of v_mfma_f32_16x16x32_bf16.  The weights stay in the packed
// tile layout of m3_pack: one 16-byte load per lane of a 1 KB tile is
// exactly the MFMA B operand (column = row l % 16 of the block, k = 8 (l /
// 16) .. +7), so weight fragments go from memory straight to registers.  The
// A tile (128 rows x 64 K) is staged in LDS, double-buffered; the next K
// step's A and weight loads are issued before the current step's MFMAs.
// Tile order: workgroups are handed to the 8 XCDs in turn, so the mapping
// puts the M tiles of one N tile on one XCD in neighbouring slots, where
// they share that XCD's L2 for the weight tiles.
//
// RMSNorm rows: one workgroup per row, a = bf16((x * r) * gamma) with r =
// 1 / sqrt(mean x^2 + eps) in fp32, the same arithmetic as the GEMV prologue.
#include "gemv_impl.h"

namespace m3 {
namespace {

constexpr int kPM = 128, kPN = 128, kPK = 64;   // workgroup tile of Y, K step
constexpr int kPThreads = 256;                  // 4 waves: 2 (M) x 2 (N) of 64 x 64
constexpr int kALd = kPK + 8;                   // LDS row stride of the A tile (bf16)

struct PrefillParams {
  const uint16_t* a;
  int lda;
  const uint8_t* w;
  uint32_t wbytes;
  uint32_t bbytes;      // bytes per packed row block
  int M, N, K;
  void* y;
  int ldy, out_f32, epi;
  const uint16_t* res;
  int ldr;
  int mtiles, ntiles;
};

// workgroup -> (M tile, N tile), XCD-aware (see above)
__device__ __forceinline__ void tile_of(const PrefillParams& p, int& mt, int& nt) {
  const int nwg = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  int logical = slot;
  for (int x = 0; x < xcd; ++x) logical += (nwg - x + 7) >> 3;   // workgroups on XCD x
  mt = logical % p.mtiles;
  nt = logical / p.mtiles;
}

template <int EPI>
__global__ __launch_bounds__(kPThreads) void prefill_gemm_kernel(PrefillParams p) {
  __shared__ __align__(16) uint16_t As[2][kPM * kALd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  int mt, nt;
  tile_of(p, mt, nt);
  const int m0 = mt * kPM, n0 = nt * kPN;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(p.w, p.wbytes);
  const int rb0 = (n0 + wn * 64) >> 4;          // this wave's first row block
  const int nk = p.K / kPK;

  // A tile (128 x 64 bf16): 1024 chunks of 16 B, 4 per thread, rows past M zero
  uint4 areg[4];
  auto load_a = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kPThreads;
      const int r = c >> 3, cc = c & 7;
      const int m = m0 + r;
      areg[i] = m < p.M ? *reinterpret_cast<const uint4*>(p.a + (size_t)m * p.lda + ks * kPK + cc * 8)
                        : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kPThreads;
      const int r = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&As[buf][r * kALd + cc * 8]) = areg[i];
    }
  };
  // weight fragments of K step ks: 4 row blocks x 2 tiles (block past N: zeros)
  uint4 wcur[4][2], wnext[4][2];
  auto load_w = [&](uint4 (&dst)[4][2], int ks) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint32_t off = (uint32_t)(rb0 + j) * p.bbytes + (uint32_t)(2 * ks + kt) * kTileBytes;
        dst[j][kt] = ldw<2>(wr, (uint32_t)lane * 16u + off, 0u);
      }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  load_w(wcur, 0);
  store_a(0);
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) {
      load_a(ks + 1);
      load_w(wnext, ks + 1);
    }
    __syncthreads();               // A tile ks is in LDS; buffer cur^1 is free
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8_t af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + (lane & 15);
        af[i] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&As[cur][r * kALd + kt * 32 + 8 * (lane >> 4)]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wcur[j][kt]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw, acc[i][j], 0, 0, 0);
      }
    }
    if (more) {
      store_a(cur ^ 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) wcur[j][kt] = wnext[j][kt];
    }
  }

  // epilogue: lane holds D[4 (l / 16) + q][l % 16] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        const int n = n0 + wn * 64 + j * 16 + (lane & 15);
        const float v = acc[i][j][q];
        if constexpr (EPI == M3_EPI_SWIGLU) {
          // interleaved gate/up rows: columns 2c (gate) and 2c+1 (up) are
          // neighbouring lanes; the even lane writes column c of the output
          const float partner = dpp_f<0xB1>(v);
          if ((lane & 1) == 0 && m < p.M && n + 1 < p.N) {
            const float g = bf2f(f2bf(v)), u = bf2f(f2bf(partner));
            const float s = g / (1.0f + expf(-g));
            reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + (n >> 1)] = (uint16_t)f2bf(s * u);
          }
        } else {
          if (m < p.M && n < p.N) {
            if (EPI == M3_EPI_RESIDUAL) {
              const uint32_t o = f2bf(bf2f(p.res[(size_t)m * p.ldr + n]) + bf2f(f2bf(v)));
              reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + n] = (uint16_t)o;
            } else if (p.out_f32) {
              reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + n] = v;
            } else {
              reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.ldy + n] = (uint16_t)f2bf(v);
            }
          }
        }
      }
}

constexpr int kNThreads = 256;

__global__ __launch_bounds__(kNThreads) void rmsnorm_rows_kernel(const uint16_t* x, int ldx,
                                                                 const float* gamma, float eps,
                                                                 int K, uint16_t* a, int lda) {
  __shared__ float part[kNThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = x + (size_t)row * ldx;
  uint16_t* ar = a + (size_t)row * lda;
  const int kc = K >> 3;
  float ss = 0.f;
  for (int c = tid; c < kc; c += kNThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c * 8);
    ss = dot2(v.x, v.x, ss);
    ss = dot2(v.y, v.y, ss);
    ss = dot2(v.z, v.z, ss);
    ss = dot2(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)K + eps);
  for (int c = tid; c < kc; c += kNThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c * 8);
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + c * 8);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + c * 8 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = (bf2f(wv[j] & 0xffffu) * r) * g[2 * j];
      const float a1 = (bf2f(wv[j] >> 16) * r) * g[2 * j + 1];
      o[j] = f2bf_pair(a0, a1);
    }
    *reinterpret_cast<uint4*>(ar + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_prefill_gemm(const PrefillDesc& d, hipStream_t s) {
  PrefillParams p{};
  p.a = d.a;
  p.lda = d.lda;
  p.w = static_cast<const uint8_t*>(d.w);
  p.bbytes = (uint32_t)block_bytes(M3_BF16, d.K);
  p.wbytes = (uint32_t)((size_t)n_blocks(d.N) * p.bbytes);
  p.M = d.M;
  p.N = d.N;
  p.K = d.K;
  p.y = d.y;
  p.ldy = d.ldy;
  p.out_f32 = d.out_f32;
  p.epi = d.epi;
  p.res = d.res;
  p.ldr = d.ldr;
  p.mtiles = (d.M + kPM - 1) / kPM;
  p.ntiles = (d.N + kPN - 1) / kPN;
  const int grid = p.mtiles * p.ntiles;
  if (d.epi == M3_EPI_SWIGLU)
    hipLaunchKernelGGL(prefill_gemm_kernel<M3_EPI_SWIGLU>, dim3(grid), dim3(kPThreads), 0, s, p);
  else if (d.epi == M3_EPI_RESIDUAL)
    hipLaunchKernelGGL(prefill_gemm_kernel<M3_EPI_RESIDUAL>, dim3(grid), dim3(kPThreads), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_gemm_kernel<M3_EPI_NONE>, dim3(grid), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const uint16_t* x, int M, int K, int ldx, const float* gamma,
                               float eps, uint16_t* a, int lda, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(M), dim3(kNThreads), 0, s, x, ldx, gamma, eps, K, a,
                     lda);
  return hipGetLastError();
}

}  // namespace m3
