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
// Attention.  A workgroup takes one (batch row, KV head, chunk of 64 or 128
// positions) and issues all of the chunk's key and value loads up front.
// Pass 1: four lanes per position, each holding 32 of the 128 dimensions as
// bf16 pairs; v_dot2 products against the G query heads of the KV head, a
// two-step DPP sum, the scores (base 2, scale folded in) to LDS.  One wave
// per head then takes the chunk's maximum, exponentials and sum.  Pass 2:
// each lane owns 4 dimensions of CH / 8 positions (a wave load reads two
// whole value rows) and accumulates P.V; the 8 half-wave partials are summed
// in LDS.  With one chunk the result is the output; otherwise (maximum, sum,
// P.V) goes to the workspace and attn_merge_kernel combines the chunks in
// order.  (Merging in the last workgroup to finish, behind an atomic count,
// measured ten times slower: the device-scope fences it needs write back and
// invalidate the L2 under every other workgroup.)  The bound is HBM: each
// position's key and value are read once (512 bytes per KV head and batch
// row).
#include "gemv_impl.h"

namespace m3 {
namespace {

constexpr int kHD = 128;
constexpr int kAThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__global__ void rope_table_kernel(float* t, int max_pos, int half, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= max_pos * half) return;
  const int p = idx / half, i = idx % half;
  const double ang = (double)p * pow(theta, -(double)i / (double)half);
  t[2 * idx] = (float)cos(ang);
  t[2 * idx + 1] = (float)sin(ang);
}

// position of a frame-driven call: pos0 + the frame counter, held below
// max_pos (a frame past the cache rewrites the last slot and flags err)
__device__ __forceinline__ int frame_pos(const uint32_t* frame_dev, int pos0, int max_pos,
                                         uint32_t* err) {
  const long p = (long)pos0 + (long)*frame_dev;
  if (p < max_pos) return (int)p;
  if (err && threadIdx.x == 0) atomicOr(err, M3_ERR_ATTN_FULL);
  return max_pos - 1;
}

// One wave per head: lane l holds elements l and l + 64 (a rotation pair).
// Row r belongs to cache sequence r / P at position pos + r % P (P = 1: one
// position for every row).  frame_dev (optional, P = 1): the position is
// pos0 + *frame_dev instead of pos.
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv, const float* q_gamma,
    const float* k_gamma, float eps, const float* rope, int pos, uint16_t* q_out, int ldq,
    uint16_t* k_cache, uint16_t* v_cache, int max_pos, const uint32_t* frame_dev, int pos0,
    uint32_t* err, int P) {
  const int heads = n_q + 2 * n_kv;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= B * heads) return;
  if (frame_dev) pos = frame_pos(frame_dev, pos0, max_pos, blockIdx.x == 0 ? err : nullptr);
  const int row = w / heads, hh = w % heads;
  const int b = row / P;                          // cache sequence
  pos += row % P;
  const uint16_t* x = qkv + (size_t)row * ldqkv + (size_t)hh * kHD;
  const uint32_t x0 = x[lane], x1 = x[lane + 64];
  if (hh >= n_q + n_kv) {                         // v: copied into the cache
    uint16_t* dst = v_cache + (((size_t)b * n_kv + (hh - n_q - n_kv)) * max_pos + pos) * kHD;
    dst[lane] = (uint16_t)x0;
    dst[lane + 64] = (uint16_t)x1;
    return;
  }
  // the head's RMSNorm with the GEMV prologue's steps (gemv_impl.h, "RMSNorm"):
  // r from a float64 sum of squares, rounded to fp32; two fp32 products
  const float* g = hh < n_q ? q_gamma : k_gamma;
  const float a0f = bf2f(x0), a1f = bf2f(x1);
  const float r = norm_r(wave_sum_f64((double)a0f * a0f + (double)a1f * a1f), kHD, eps);
  const float a0 = bf2f(f2bf((a0f * r) * g[lane])), a1 = bf2f(f2bf((a1f * r) * g[lane + 64]));
  const float c = rope[((size_t)pos * 64 + lane) * 2], s = rope[((size_t)pos * 64 + lane) * 2 + 1];
  const uint32_t y0 = f2bf(a0 * c - a1 * s), y1 = f2bf(a1 * c + a0 * s);
  uint16_t* dst = hh < n_q ? q_out + (size_t)row * ldq + (size_t)hh * kHD
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
  float* ws;                                     // [B][n_kv][nchunks][G][2 + 128]
  const uint32_t* frame_dev;                     // optional: T = pos0 + *frame_dev + 1
  int pos0;
  int ch;                                        // positions per chunk
  int P;                                         // rows per cache sequence
  int T0;                                        // positions attended by a sequence's first row
};

// positions attended by row r: T0 + r % P (row r of cache sequence r / P; P =
// 1 and T0 = T for one position per row), or the frame's position + 1 (grid
// and records are sized for p.T = max_pos then)
__device__ __forceinline__ int attn_T(const AttnParams& p, int r) {
  if (!p.frame_dev) return p.T0 + r % p.P;
  const long t = (long)p.pos0 + (long)*p.frame_dev + 1;
  return t < p.max_pos ? (int)t : p.max_pos;
}

template <int G, int CH>
__global__ __launch_bounds__(kAThreads) void attn_kernel(AttnParams p) {
  constexpr int PJ = CH / 64;                    // pass-1 positions per 4-lane group
  constexpr int PI = CH / 8;                     // pass-2 positions per lane
  constexpr int WP = CH / 4;                     // pass-2 positions per wave
  __shared__ __align__(16) float S[CH][G];       // scores, then probabilities
  __shared__ float Ms[G], Ls[G];
  __shared__ __align__(16) float pacc[8][G][kHD];   // P.V partials of the 8 half-waves
  const int chunk = blockIdx.x % p.nchunks;
  const int kvh = (blockIdx.x / p.nchunks) % p.n_kv;
  const int b = blockIdx.x / (p.nchunks * p.n_kv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = attn_T(p, b), nc = (T + CH - 1) / CH;
  if (chunk >= nc) return;                       // past this row's position
  const int t0 = chunk * CH;
  const int n = min(T - t0, CH);                 // positions of this chunk
  const size_t base = ((size_t)(b / p.P) * p.n_kv + kvh) * (size_t)p.max_pos * kHD;
  const uint16_t* kb = p.k + base;
  const uint16_t* vb = p.v + base;

  // pass 1 layout: a group of 4 lanes per position, lane li holding the
  // 16-byte chunks 4 c + li (c < 4) of the row: positions grp + 64 j
  const int grp = tid >> 2, li = tid & 3;
  // loads retire in issue order: q first, then the keys pass 1 needs, then
  // the values pass 2 needs
  uint4 qr[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qr[h][c] = *reinterpret_cast<const uint4*>(p.q + (size_t)b * p.ldq + (size_t)(kvh * G + h) * kHD +
                                                 8 * (4 * c + li));
  uint4 kr[PJ][4];
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int t = t0 + min(grp + 64 * j, n - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kr[j][c] = *reinterpret_cast<const uint4*>(kb + (size_t)t * kHD + 8 * (4 * c + li));
  }
  // pass 2 layout: lane owns dimensions 4 dq .. 4 dq + 3 of positions
  // WP w + 2 i + sub (i < PI), so a wave load reads two whole rows
  const int dq = lane & 31, sub = lane >> 5;
  uint2 vr[PI];
#pragma unroll
  for (int i = 0; i < PI; ++i) {
    const int t = t0 + min(WP * wave + 2 * i + sub, n - 1);
    vr[i] = *reinterpret_cast<const uint2*>(vb + (size_t)t * kHD + 4 * dq);
  }

  // pass 1: scores (base 2, scale folded in); masked positions get -inf
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int tc = grp + 64 * j;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s = dot2(qr[h][c].x, kr[j][c].x, s);
        s = dot2(qr[h][c].y, kr[j][c].y, s);
        s = dot2(qr[h][c].z, kr[j][c].z, s);
        s = dot2(qr[h][c].w, kr[j][c].w, s);
      }
      s += dpp_f<0xB1>(s);                       // the 4 lanes of the group
      s += dpp_f<0x4E>(s);
      if (li == 0) S[tc][h] = tc < n ? s * p.scale2 : -INFINITY;
    }
  }
  __syncthreads();
  // softmax over the chunk, one wave per head
  for (int h = wave; h < G; h += 4) {
    float e[PJ], m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PJ; ++j) m = fmaxf(m, S[lane + 64 * j][h]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      e[j] = exp2f(S[lane + 64 * j][h] - m);
      S[lane + 64 * j][h] = e[j];
      l += e[j];
    }
    l = wave_sum(l);
    if (lane == 0) {
      Ms[h] = m;
      Ls[h] = l;
    }
  }
  __syncthreads();
  // pass 2: P.V over this lane's positions and 4 dimensions
  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < PI; ++i) {
    const int tc = WP * wave + 2 * i + sub;
    const float v0 = bf2f(vr[i].x & 0xffffu), v1 = bf2f(vr[i].x >> 16);
    const float v2 = bf2f(vr[i].y & 0xffffu), v3 = bf2f(vr[i].y >> 16);
    float prs[G];                                // 0 for masked positions
#pragma unroll
    for (int h = 0; h < G; ++h) prs[h] = S[tc][h];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = prs[h];
      acc[h][0] = fmaf(pr, v0, acc[h][0]);
      acc[h][1] = fmaf(pr, v1, acc[h][1]);
      acc[h][2] = fmaf(pr, v2, acc[h][2]);
      acc[h][3] = fmaf(pr, v3, acc[h][3]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
    *reinterpret_cast<float4*>(&pacc[2 * wave + sub][h][4 * dq]) =
        make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  __syncthreads();
  float* wrec = p.ws + (((size_t)b * p.n_kv + kvh) * p.nchunks) * (G * (2 + kHD));
  for (int o = tid; o < G * kHD; o += kAThreads) {
    const int h = o / kHD, d = o % kHD;
    float A = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) A += pacc[k][h][d];
    if (nc == 1) {
      p.out[(size_t)b * p.ldo + (size_t)(kvh * G + h) * kHD + d] = (uint16_t)f2bf(A / Ls[h]);
    } else {
      float* w = wrec + ((size_t)chunk * G + h) * (2 + kHD);
      if (d == 0) {
        w[0] = Ms[h];
        w[1] = Ls[h];
      }
      w[2 + d] = A;
    }
  }
}

// chunks combined in order: one workgroup of 128 threads per (row, query
// head).  Every load of a batch of up to 32 chunks (their maxima, sums and
// this thread's P.V dimension) is issued before the first is used, so a
// merge of up to 32 chunks (2048 or 4096 positions) waits for memory once.
constexpr int kMergeBatch = 32;

template <int G>
__global__ __launch_bounds__(kHD) void attn_merge_kernel(AttnParams p) {
  const int qh = blockIdx.x % p.n_q, b = blockIdx.x / p.n_q, d = threadIdx.x;
  const int kvh = qh / G, h = qh % G;
  const int nc = (attn_T(p, b) + p.ch - 1) / p.ch;
  if (nc == 1) return;                           // the chunk kernel wrote the output
  const float* wrec = p.ws + (((size_t)b * p.n_kv + kvh) * p.nchunks) * (G * (2 + kHD)) + h * (2 + kHD);
  constexpr size_t kStride = (size_t)G * (2 + kHD);   // floats from one chunk's record to the next
  float mv[kMergeBatch], lv[kMergeBatch], av[kMergeBatch];
  auto load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool in = c0 + u < nc;
      const float* wc = wrec + (c0 + u) * kStride;
      mv[u] = in ? wc[0] : -INFINITY;
      lv[u] = in ? wc[1] : 0.f;
      av[u] = in ? wc[2 + d] : 0.f;
    }
  };
  float M = -INFINITY, L = 0.f, A = 0.f;
  auto add = [&]() {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float e = exp2f(mv[u] - M);          // 0 past the last chunk
      L = fmaf(lv[u], e, L);
      A = fmaf(av[u], e, A);
    }
  };
  if (nc <= kMergeBatch) {                       // one batch: a single wait for memory
    load(0);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) M = fmaxf(M, mv[u]);
    add();
  } else {                                       // the maximum over every chunk first
    for (int c0 = 0; c0 < nc; c0 += kMergeBatch)
      for (int c = c0; c < min(nc, c0 + kMergeBatch); ++c) M = fmaxf(M, wrec[c * kStride]);
    for (int c0 = 0; c0 < nc; c0 += kMergeBatch) {
      load(c0);
      add();
    }
  }
  p.out[(size_t)b * p.ldo + (size_t)qh * kHD + d] = (uint16_t)f2bf(A / L);
}

template <int G>
void launch_attn_g(const AttnParams& p, int CH, int B, hipStream_t s) {
  const dim3 grid(B * p.n_kv * p.nchunks);
  if (CH == 64)
    hipLaunchKernelGGL((attn_kernel<G, 64>), grid, dim3(kAThreads), 0, s, p);
  else
    hipLaunchKernelGGL((attn_kernel<G, 128>), grid, dim3(kAThreads), 0, s, p);
  if (p.nchunks > 1) hipLaunchKernelGGL((attn_merge_kernel<G>), dim3(B * p.n_q), dim3(kHD), 0, s, p);
}

}  // namespace

// positions per workgroup: 128, or 64 where 128 would leave most CUs idle
int attn_chunk_size(int B, int n_kv, int T) {
  return (size_t)B * n_kv * ((T + 127) / 128) < 256 ? 64 : 128;
}

size_t attn_workspace_bytes(int B, int n_q, int n_kv, int T) {
  const int ch = attn_chunk_size(B, n_kv, T), nc = (T + ch - 1) / ch;
  return nc == 1 ? 0 : (size_t)B * n_q * nc * (2 + kHD) * sizeof(float);
}

hipError_t launch_rope_table(float* t, int max_pos, int head_dim, double theta, hipStream_t s) {
  const int half = head_dim / 2, n = max_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, t, max_pos, half,
                     theta);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                               const float* q_gamma, const float* k_gamma, float eps,
                               const float* rope, int pos, uint16_t* q_out, int ldq,
                               uint16_t* k_cache, uint16_t* v_cache, int max_pos, hipStream_t s,
                               const uint32_t* frame_dev, int pos0, uint32_t* err, int P) {
  const int waves = B * (n_q + 2 * n_kv);
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, qkv, B, ldqkv,
                     n_q, n_kv, q_gamma, k_gamma, eps, rope, pos, q_out, ldq, k_cache, v_cache,
                     max_pos, frame_dev, pos0, err, P);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const uint16_t* q, int B, int ldq, int n_q, int n_kv,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                                   int T, uint16_t* out, int ldo, void* ws, hipStream_t s,
                                   const uint32_t* frame_dev, int pos0, int P) {
  // the grid and the records are sized for the longest row: T + P - 1, or
  // every position for a frame-driven call
  const int Tg = frame_dev ? max_pos : T + P - 1;
  const int ch = attn_chunk_size(B, n_kv, Tg);
  const int nc = (Tg + ch - 1) / ch;
  AttnParams p{q, ldq, k_cache, v_cache, n_q, n_kv, max_pos, Tg, nc, kLog2e / sqrtf((float)kHD),
               out, ldo, static_cast<float*>(ws), frame_dev, pos0, ch, P, T};
  switch (n_q / n_kv) {
    case 1: launch_attn_g<1>(p, ch, B, s); break;
    case 2: launch_attn_g<2>(p, ch, B, s); break;
    case 4: launch_attn_g<4>(p, ch, B, s); break;
    default: launch_attn_g<8>(p, ch, B, s); break;
  }
  return hipGetLastError();
}

}  // namespace m3
