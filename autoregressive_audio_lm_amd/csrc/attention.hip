// attention.hip -- decode attention in place of the identity stub: the RoPE
// table, per-head q/k RMSNorm + RoPE with the KV-cache writes, and softmax
// attention of one new query row per batch row over the cached positions.
//
// "MiniMax Music 3, local" and TensorFold PR #987 list these steps among the
// decode kernels: a per-head q/k norm and RoPE, decode attention that splits
// the keys and merges the partial softmax sums, and the depth decoder's
// attention over its codebook positions; the precision contract there keeps
// norms, RoPE, softmax and attention sums in fp32 over bf16 activations.
// The body is Qwen3-shaped: head_dim 128, RoPE base 1e6 rotating the pairs
// (i, i + 64), 32 query heads over 8 KV heads; the depth decoder has 16:16.
//
// Cache layout (bf16): [B][n_kv][max_pos][128], so the keys of one KV head
// are contiguous rows of 256 bytes.
//
// Attention.  A workgroup takes one (batch row, KV head, chunk of kChunk
// positions).  A wave is four groups of 16 lanes; a group owns one position
// at a time and a lane 8 of its 128 dimensions (one 16-byte load), so a wave
// load covers four neighbouring cache rows, 1 KB contiguous.  The group's
// score for each of the G query heads of the KV head is a 16-lane DPP row
// sum; the group keeps a running maximum, sum and weighted V (online
// softmax in base 2) over its positions.  The 16 group states of the
// workgroup are merged in LDS; with one chunk the result is the output,
// otherwise it goes to the workspace and attn_merge_kernel combines the
// chunks in order.  The bound is HBM: each position's key and value are read
// once (512 bytes per KV head and batch row).
#include "gemv_impl.h"

namespace m3 {
namespace {

constexpr int kHD = 128;
constexpr int kChunk = 128;                      // positions per workgroup
constexpr int kAThreads = 256;
constexpr int kGroups = kAThreads / 16;          // 16-lane groups per workgroup
constexpr int kPerGroup = kChunk / kGroups;      // positions per group
constexpr float kLog2e = 1.4426950408889634f;

// sum over the 16 lanes of a DPP row
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);     // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);    // row_half_mirror
  v += dpp_f<0x140>(v);    // row_mirror
  return v;
}

__global__ void rope_table_kernel(float* t, int max_pos, int half, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= max_pos * half) return;
  const int p = idx / half, i = idx % half;
  const double ang = (double)p * pow(theta, -(double)i / (double)half);
  t[2 * idx] = (float)cos(ang);
  t[2 * idx + 1] = (float)sin(ang);
}

// One wave per head: lane l holds elements l and l + 64 (a rotation pair).
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv, const float* q_gamma,
    const float* k_gamma, float eps, const float* rope, int pos, uint16_t* q_out, int ldq,
    uint16_t* k_cache, uint16_t* v_cache, int max_pos) {
  const int heads = n_q + 2 * n_kv;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= B * heads) return;
  const int b = w / heads, hh = w % heads;
  const uint16_t* x = qkv + (size_t)b * ldqkv + (size_t)hh * kHD;
  const uint32_t x0 = x[lane], x1 = x[lane + 64];
  if (hh >= n_q + n_kv) {                         // v: copied into the cache
    uint16_t* dst = v_cache + (((size_t)b * n_kv + (hh - n_q - n_kv)) * max_pos + pos) * kHD;
    dst[lane] = (uint16_t)x0;
    dst[lane + 64] = (uint16_t)x1;
    return;
  }
  const float* g = hh < n_q ? q_gamma : k_gamma;
  const float a0f = bf2f(x0), a1f = bf2f(x1);
  const float tot = wave_sum(a0f * a0f + a1f * a1f);
  const float r = 1.0f / sqrtf(tot / (float)kHD + eps);
  const float a0 = bf2f(f2bf((a0f * r) * g[lane])), a1 = bf2f(f2bf((a1f * r) * g[lane + 64]));
  const float c = rope[((size_t)pos * 64 + lane) * 2], s = rope[((size_t)pos * 64 + lane) * 2 + 1];
  const uint32_t y0 = f2bf(a0 * c - a1 * s), y1 = f2bf(a1 * c + a0 * s);
  uint16_t* dst = hh < n_q ? q_out + (size_t)b * ldq + (size_t)hh * kHD
                           : k_cache + (((size_t)b * n_kv + (hh - n_q)) * max_pos + pos) * kHD;
  dst[lane] = (uint16_t)y0;
  dst[lane + 64] = (uint16_t)y1;
}

struct AttnParams {
  const uint16_t* q;
  int ldq;
  const uint16_t* k;
  const uint16_t* v;
  int n_q, n_kv, max_pos, T, nchunks;
  float scale2;                                  // log2(e) / sqrt(head_dim)
  uint16_t* out;
  int ldo;
  float* ws;                                     // [B][n_q][nchunks][2 + 128]
};

template <int G>
__global__ __launch_bounds__(kAThreads) void attn_partial_kernel(AttnParams p) {
  __shared__ float sm[kGroups][G], sl[kGroups][G];
  __shared__ float sacc[kGroups][G][kHD];
  const int chunk = blockIdx.x % p.nchunks;
  const int kvh = (blockIdx.x / p.nchunks) % p.n_kv;
  const int b = blockIdx.x / (p.nchunks * p.n_kv);
  const int tid = threadIdx.x, lane = tid & 63, grp = tid >> 4, ds = lane & 15;
  const int t0 = chunk * kChunk;
  const int t_end = min(p.T, t0 + kChunk);

  // this lane's 8 dimensions of the G query heads, in fp32
  float q[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 u = *reinterpret_cast<const uint4*>(p.q + (size_t)b * p.ldq +
                                                     (size_t)(kvh * G + h) * kHD + 8 * ds);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[h][2 * j] = bf2f(w[j] & 0xffffu);
      q[h][2 * j + 1] = bf2f(w[j] >> 16);
    }
  }
  // the group's positions: t0 + grp + kGroups * j (a wave's four groups read
  // four neighbouring rows); loads are clamped into [0, T) and masked below
  const size_t base = ((size_t)b * p.n_kv + kvh) * (size_t)p.max_pos * kHD + 8 * ds;
  uint4 kr[kPerGroup], vr[kPerGroup];
#pragma unroll
  for (int j = 0; j < kPerGroup; ++j) {
    const int t = min(t0 + grp + kGroups * j, p.T - 1);
    kr[j] = *reinterpret_cast<const uint4*>(p.k + base + (size_t)t * kHD);
    vr[j] = *reinterpret_cast<const uint4*>(p.v + base + (size_t)t * kHD);
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kPerGroup; ++j) {
    if (t0 + grp + kGroups * j >= t_end) break;  // uniform within the group
    const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
    const uint32_t vw[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[2 * e] = bf2f(kw[e] & 0xffffu);
      kf[2 * e + 1] = bf2f(kw[e] >> 16);
      vf[2 * e] = bf2f(vw[e] & 0xffffu);
      vf[2 * e + 1] = bf2f(vw[e] >> 16);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) s = fmaf(q[h][d], kf[d], s);
      s = row16_sum(s) * p.scale2;
      const float mn = fmaxf(m[h], s);
      const float corr = exp2f(m[h] - mn), pr = exp2f(s - mn);
      m[h] = mn;
      l[h] = l[h] * corr + pr;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] = fmaf(pr, vf[d], acc[h][d] * corr);
    }
  }
  // the 16 group states of the workgroup, merged in LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (ds == 0) {
      sm[grp][h] = m[h];
      sl[grp][h] = l[h];
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) sacc[grp][h][8 * ds + d] = acc[h][d];
  }
  __syncthreads();
  for (int o = tid; o < G * kHD; o += kAThreads) {
    const int h = o / kHD, d = o % kHD;
    float M = -INFINITY;
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) M = fmaxf(M, sm[gi][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const float e = sm[gi][h] == -INFINITY ? 0.f : exp2f(sm[gi][h] - M);
      L = fmaf(sl[gi][h], e, L);
      A = fmaf(sacc[gi][h][d], e, A);
    }
    const int qh = kvh * G + h;
    if (p.nchunks == 1) {
      p.out[(size_t)b * p.ldo + (size_t)qh * kHD + d] = (uint16_t)f2bf(A / L);
    } else {
      float* w = p.ws + (((size_t)b * p.n_q + qh) * p.nchunks + chunk) * (2 + kHD);
      if (d == 0) {
        w[0] = M;
        w[1] = L;
      }
      w[2 + d] = A;
    }
  }
}

// chunks combined in order: one workgroup of 128 threads per (row, head)
__global__ __launch_bounds__(kHD) void attn_merge_kernel(AttnParams p) {
  const int qh = blockIdx.x % p.n_q, b = blockIdx.x / p.n_q, d = threadIdx.x;
  const float* w = p.ws + ((size_t)b * p.n_q + qh) * p.nchunks * (2 + kHD);
  float M = -INFINITY;
  for (int c = 0; c < p.nchunks; ++c) M = fmaxf(M, w[c * (2 + kHD)]);
  float L = 0.f, A = 0.f;
  for (int c = 0; c < p.nchunks; ++c) {
    const float* wc = w + c * (2 + kHD);
    const float e = wc[0] == -INFINITY ? 0.f : exp2f(wc[0] - M);
    L = fmaf(wc[1], e, L);
    A = fmaf(wc[2 + d], e, A);
  }
  p.out[(size_t)b * p.ldo + (size_t)qh * kHD + d] = (uint16_t)f2bf(A / L);
}

}  // namespace

int attn_chunks(int T) { return (T + kChunk - 1) / kChunk; }

hipError_t launch_rope_table(float* t, int max_pos, int head_dim, double theta, hipStream_t s) {
  const int half = head_dim / 2, n = max_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, t, max_pos, half,
                     theta);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                               const float* q_gamma, const float* k_gamma, float eps,
                               const float* rope, int pos, uint16_t* q_out, int ldq,
                               uint16_t* k_cache, uint16_t* v_cache, int max_pos, hipStream_t s) {
  const int waves = B * (n_q + 2 * n_kv);
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, qkv, B, ldqkv,
                     n_q, n_kv, q_gamma, k_gamma, eps, rope, pos, q_out, ldq, k_cache, v_cache,
                     max_pos);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const uint16_t* q, int B, int ldq, int n_q, int n_kv,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                                   int T, uint16_t* out, int ldo, float* ws, hipStream_t s) {
  AttnParams p{q, ldq, k_cache, v_cache, n_q, n_kv, max_pos, T, attn_chunks(T),
               kLog2e / sqrtf((float)kHD), out, ldo, ws};
  const dim3 grid(B * n_kv * p.nchunks);
  switch (n_q / n_kv) {
    case 1: hipLaunchKernelGGL(attn_partial_kernel<1>, grid, dim3(kAThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(attn_partial_kernel<2>, grid, dim3(kAThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(attn_partial_kernel<4>, grid, dim3(kAThreads), 0, s, p); break;
    default: hipLaunchKernelGGL(attn_partial_kernel<8>, grid, dim3(kAThreads), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nchunks == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(B * n_q), dim3(kHD), 0, s, p);
  return hipGetLastError();
}

}  // namespace m3
