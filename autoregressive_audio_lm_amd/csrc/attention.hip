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
// positions) and issues all of the chunk's query, key and value loads up
// front; the chunk's arithmetic is attn_compute (attn_impl.h).  With one
// chunk the result is the output; otherwise (maximum, sum, P.V) goes to the
// workspace and attn_merge_kernel combines the chunks in order.  (Merging in
// the last workgroup to finish, behind an atomic count, measured ten times
// slower: the device-scope fences it needs write back and invalidate the L2
// under every other workgroup.)  The bound is HBM: each position's key and
// value are read once (512 bytes per KV head and batch row).
#include "attn_impl.h"

namespace m3 {
namespace {

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
  // the head's RMSNorm with the GEMV prologue's steps, then RoPE
  const float* g = hh < n_q ? q_gamma : k_gamma;
  uint32_t y0, y1;
  head_norm_rope(x0, x1, g, eps, rope, pos, lane, y0, y1);
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
  __shared__ AttnLds<G, CH> L;
  const int chunk = blockIdx.x % p.nchunks;
  const int kvh = (blockIdx.x / p.nchunks) % p.n_kv;
  const int b = blockIdx.x / (p.nchunks * p.n_kv);
  const int tid = threadIdx.x;
  const int T = attn_T(p, b), nc = (T + CH - 1) / CH;
  if (chunk >= nc) return;                       // past this row's position
  const int t0 = chunk * CH;
  const int n = min(T - t0, CH);                 // positions of this chunk
  const size_t base = ((size_t)(b / p.P) * p.n_kv + kvh) * (size_t)p.max_pos * kHD;
  // loads retire in issue order: q first, then the keys pass 1 needs, then
  // the values pass 2 needs
  AttnRegs<G, CH> R;
  attn_load_q(R, p.q + (size_t)b * p.ldq + (size_t)kvh * G * kHD, tid);
  attn_load_kv(R, p.k + base, p.v + base, t0, n, tid);
  float* wrec = p.ws + (((size_t)b * p.n_kv + kvh) * p.nchunks) * (G * (2 + kHD));
  attn_compute(R, n, p.scale2, tid, L, [&](int h, int d, float A, float M, float Lh) {
    if (nc == 1) {
      p.out[(size_t)b * p.ldo + (size_t)(kvh * G + h) * kHD + d] = (uint16_t)f2bf(A / Lh);
    } else {
      float* w = wrec + ((size_t)chunk * G + h) * (2 + kHD);
      if (d == 0) {
        w[0] = M;
        w[1] = Lh;
      }
      w[2 + d] = A;
    }
  });
}

// The frame's attention step in one launch: q/k norm + RoPE, the cache write
// and the chunk's partial softmax (the arithmetic of qk_norm_rope_kernel and
// attn_kernel, so the results are theirs).  Workgroup (row, KV head, chunk)
// first requests its chunk's cached keys and values, then norms and rotates
// its G query heads from the QKV row into LDS; the chunk holding the position
// also norms and rotates that position's key and writes key and value to the
// cache, and takes them from LDS (the other cached rows were written by
// earlier launches).  One position per row (P = 1).
struct FusedAttn {
  AttnParams p;                 // q and ldq unused
  const uint16_t* qkv;
  int ldqkv;
  const float *q_gamma, *k_gamma, *rope;
  float eps;
  int pos;                      // without frame_dev
  uint16_t *k_cache, *v_cache;
  uint32_t* err;
};

template <int G, int CH>
__global__ __launch_bounds__(kAThreads) void attn_fused_kernel(FusedAttn f) {
  __shared__ AttnLds<G, CH> L;
  __shared__ __align__(16) uint16_t qs[(G + 2) * kHD];   // q heads, then the position's k, v
  const AttnParams& p = f.p;
  const int chunk = blockIdx.x % p.nchunks;
  const int kvh = (blockIdx.x / p.nchunks) % p.n_kv;
  const int b = blockIdx.x / (p.nchunks * p.n_kv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos = p.frame_dev ? frame_pos(p.frame_dev, p.pos0, p.max_pos, blockIdx.x == 0 ? f.err : nullptr)
                              : f.pos;
  const int T = pos + 1, nc = (T + CH - 1) / CH;
  if (chunk >= nc) return;                       // past this row's position
  const int t0 = chunk * CH;
  const int n = min(T - t0, CH);
  const bool last = chunk == nc - 1;
  const size_t base = ((size_t)b * p.n_kv + kvh) * (size_t)p.max_pos * kHD;
  uint16_t* kb = f.k_cache + base;
  uint16_t* vb = f.v_cache + base;
  AttnRegs<G, CH> R;
  attn_load_kv(R, kb, vb, t0, n, tid);
  uint16_t* kvs = qs + G * kHD;
  for (int k = wave; k < G + (last ? 2 : 0); k += 4) {
    const int head = k < G ? kvh * G + k : (k == G ? p.n_q + kvh : p.n_q + p.n_kv + kvh);
    const uint16_t* x = f.qkv + (size_t)b * f.ldqkv + (size_t)head * kHD;
    uint32_t y0 = x[lane], y1 = x[lane + 64];
    if (k <= G)
      head_norm_rope(y0, y1, k < G ? f.q_gamma : f.k_gamma, f.eps, f.rope, pos, lane, y0, y1);
    uint16_t* dst = k < G ? qs + k * kHD : kvs + (k - G) * kHD;
    dst[lane] = (uint16_t)y0;
    dst[lane + 64] = (uint16_t)y1;
    if (k >= G) {
      uint16_t* c = (k == G ? kb : vb) + (size_t)pos * kHD;
      c[lane] = (uint16_t)y0;
      c[lane + 64] = (uint16_t)y1;
    }
  }
  __syncthreads();
  if (last) attn_set_kv_at(R, kvs, kvs + kHD, t0, n, tid, pos);
  float* wrec = p.ws + (((size_t)b * p.n_kv + kvh) * p.nchunks) * (G * (2 + kHD));
  attn_compute(R, n, p.scale2, tid, L, [&](int h, int d, float A, float M, float Lh) {
    if (nc == 1) {
      p.out[(size_t)b * p.ldo + (size_t)(kvh * G + h) * kHD + d] = (uint16_t)f2bf(A / Lh);
    } else {
      float* w = wrec + ((size_t)chunk * G + h) * (2 + kHD);
      if (d == 0) {
        w[0] = M;
        w[1] = Lh;
      }
      w[2 + d] = A;
    }
  }, qs);
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

template <int G>
void launch_fused_g(const FusedAttn& f, int CH, int B, hipStream_t s) {
  const dim3 grid(B * f.p.n_kv * f.p.nchunks);
  if (CH == 64)
    hipLaunchKernelGGL((attn_fused_kernel<G, 64>), grid, dim3(kAThreads), 0, s, f);
  else
    hipLaunchKernelGGL((attn_fused_kernel<G, 128>), grid, dim3(kAThreads), 0, s, f);
  if (f.p.nchunks > 1)
    hipLaunchKernelGGL((attn_merge_kernel<G>), dim3(B * f.p.n_q), dim3(kHD), 0, s, f.p);
}


// ---------------------------------------------------------------------------
// Prompt attention, tiled.  One workgroup per (sequence, KV head, block of RB
// prompt rows) holds the 64 query vectors of those rows' G heads (vector v =
// row t0 + v / G, head G kvh + v % G) and walks the keys 0 .. the block's last
// position in chunks of 64, keeping a running maximum, sum and P.V per vector:
// no partial records and no merge.  Scores: v_mfma_f32_32x32x16_bf16 (bf16
// products, fp32 sums; each wave one 32 x 32 block of vectors x keys, q in
// registers, keys straight from the cache), scaled to base 2 and masked past
// each row's position; softmax in fp32 on the VALU and P.V on
// v_mfma_f32_32x32x2f32 (fp32 products and sums) as in the decode kernels:
// p = 2^(s - m), a new maximum rescales the sum and the P.V by
// 2^(m_old - m_new), out = bf16(P.V / sum).
constexpr int kPQ = 64;                          // query vectors per workgroup
constexpr int kPK = 64;                          // keys per chunk

typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PromptAttn {
  const uint16_t* q;
  int ldq;
  const uint16_t* k;
  const uint16_t* v;
  int n_kv, max_pos, P, pos_base, nrb;
  float scale2;                                  // log2(e) / sqrt(head_dim)
  uint16_t* out;
  int ldo;
};

template <int G>
__global__ __launch_bounds__(kAThreads, 2) void prompt_attn_kernel(PromptAttn a) {
  constexpr int RB = kPQ / G;
  __shared__ float Pt[kPK][kPQ + 1];             // scores, then probabilities: [key][vector]
  __shared__ __align__(16) uint16_t Vs[kPK][kHD];
  __shared__ float As[kPQ], Ls[kPQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int w = blockIdx.x;                            // the longest row blocks first
  const int rb = a.nrb - 1 - w % a.nrb;
  w /= a.nrb;
  const int kvh = w % a.n_kv, sq = w / a.n_kv;
  const int t0 = rb * RB;
  const int nkeys = a.pos_base + min(t0 + RB, a.P);   // keys 0 .. the block's last position
  const int nch = (nkeys + kPK - 1) / kPK;
  const size_t cb = (size_t)(sq * a.n_kv + kvh) * a.max_pos * kHD;
  const uint16_t* kb = a.k + cb;
  const uint16_t* vb = a.v + cb;
  auto vpos = [&](int v) { return a.pos_base + min(t0 + v / G, a.P - 1); };

  // scores: wave (qb, kc) = block of vectors 32 qb .., keys 32 kc .. of a chunk;
  // A operand: vector 32 qb + l % 32, dims 16 ks + 8 (l / 32) .. +7
  const int qb = wave >> 1, kc = wave & 1;
  uint4 qa[8];
  {
    const int v = 32 * qb + (lane & 31);
    const uint16_t* qr = a.q + (size_t)(sq * a.P + min(t0 + v / G, a.P - 1)) * a.ldq +
                         (size_t)(kvh * G + v % G) * kHD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qa[ks] = *reinterpret_cast<const uint4*>(qr + 16 * ks);
  }
  // the next chunk's keys (this wave's 32) and values (4 x 16 bytes per thread)
  uint4 kk[8], vv[4];
  auto load_chunk = [&](int k0) {
    const uint16_t* kr = kb + (size_t)min(k0 + 32 * kc + (lane & 31), nkeys - 1) * kHD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kk[ks] = *reinterpret_cast<const uint4*>(kr + 16 * ks);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * kAThreads, j = e >> 4, d8 = e & 15;
      vv[u] = *reinterpret_cast<const uint4*>(vb + (size_t)min(k0 + j, nkeys - 1) * kHD + 8 * d8);
    }
  };
  // softmax: 4 threads per vector, 16 keys each
  const int sv = tid >> 2, sk = tid & 3;
  float m_run = -INFINITY, l_run = 0.f;
  // P.V on v_mfma_f32_32x32x2_f32: wave (pb, dc) holds vectors 32 pb .., dims
  // 64 dc .. +63 as two 32 x 32 blocks; A = P[vector l % 32][key 2 s + l / 32],
  // B = V[key 2 s + l / 32][dim l % 32]
  const int pb = wave >> 1, dc = wave & 1;
  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

  load_chunk(0);
  for (int c = 0; c < nch; ++c) {
    const int k0 = c * kPK;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * kAThreads;
      *reinterpret_cast<uint4*>(&Vs[e >> 4][8 * (e & 15)]) = vv[u];
    }
    {
      f32x16_t sacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qa[ks]),
                                                       __builtin_bit_cast(bf16x8_t, kk[ks]), sacc, 0, 0, 0);
      // lane holds S[32 qb + 8 g + 4 (l / 32) + r][32 kc + l % 32] in sacc[4 g + r]
      const int j = 32 * kc + (lane & 31), kp = k0 + j;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = 32 * qb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        Pt[j][v] = kp < nkeys && kp <= vpos(v) ? sacc[e] * a.scale2 : -INFINITY;
      }
    }
    if (c + 1 < nch) load_chunk(k0 + kPK);       // in flight through the softmax and P.V
    __syncthreads();
    {
      float x[16], mc = -INFINITY;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        x[u] = Pt[16 * sk + u][sv];
        mc = fmaxf(mc, x[u]);
      }
      mc = fmaxf(mc, __shfl_xor(mc, 1));
      mc = fmaxf(mc, __shfl_xor(mc, 2));
      const float m_new = fmaxf(m_run, mc);      // finite: key 0 is seen by every row
      const float alpha = exp2f(m_run - m_new);  // 0 at the first chunk
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float pr = exp2f(x[u] - m_new);
        Pt[16 * sk + u][sv] = pr;
        ls += pr;
      }
      ls += __shfl_xor(ls, 1);
      ls += __shfl_xor(ls, 2);
      l_run = fmaf(l_run, alpha, ls);
      m_run = m_new;
      if (sk == 0) As[sv] = alpha;
    }
    __syncthreads();
    {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float al = As[32 * pb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)];
        acc[0][e] *= al;
        acc[1][e] *= al;
      }
      const int pv = 32 * pb + (lane & 31);
#pragma unroll 8
      for (int s2 = 0; s2 < kPK / 2; ++s2) {
        const int j = 2 * s2 + (lane >> 5);
        const float pa = Pt[j][pv];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              pa, bf2f(Vs[j][64 * dc + 32 * h + (lane & 31)]), acc[h], 0, 0, 0);
      }
    }
    __syncthreads();                             // Pt and Vs are rewritten by the next chunk
  }
  if (sk == 0) Ls[sv] = l_run;
  __syncthreads();
  // lane holds O[32 pb + 8 g + 4 (l / 32) + r][64 dc + 32 h + l % 32] in acc[h][4 g + r]
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int v = 32 * pb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), t = t0 + v / G;
    if (t >= a.P) continue;
    const float L = Ls[v];
    uint16_t* orow = a.out + (size_t)(sq * a.P + t) * a.ldo + (size_t)(kvh * G + v % G) * kHD + 64 * dc + (lane & 31);
    orow[0] = (uint16_t)f2bf(acc[0][e] / L);
    orow[32] = (uint16_t)f2bf(acc[1][e] / L);
  }
}

template <int G>
void launch_prompt_g(const PromptAttn& a, int S, hipStream_t s) {
  hipLaunchKernelGGL(prompt_attn_kernel<G>, dim3(S * a.n_kv * a.nrb), dim3(kAThreads), 0, s, a);
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

hipError_t launch_attention_fused(const uint16_t* qkv, int B, int ldqkv, int n_q, int n_kv,
                                  const float* q_gamma, const float* k_gamma, float eps,
                                  const float* rope, int pos, uint16_t* k_cache,
                                  uint16_t* v_cache, int max_pos, uint16_t* out, int ldo, void* ws,
                                  hipStream_t s, const uint32_t* frame_dev, int pos0,
                                  uint32_t* err) {
  // grid and records as the two-launch path: every position for a
  // frame-driven call, pos + 1 otherwise
  const int Tg = frame_dev ? max_pos : pos + 1;
  const int ch = attn_chunk_size(B, n_kv, Tg);
  const int nc = (Tg + ch - 1) / ch;
  FusedAttn f{};
  f.p = AttnParams{nullptr, 0, k_cache, v_cache, n_q, n_kv, max_pos, Tg, nc,
                   kLog2e / sqrtf((float)kHD), out, ldo, static_cast<float*>(ws), frame_dev, pos0,
                   ch, 1, pos + 1};
  f.qkv = qkv;
  f.ldqkv = ldqkv;
  f.q_gamma = q_gamma;
  f.k_gamma = k_gamma;
  f.rope = rope;
  f.eps = eps;
  f.pos = pos;
  f.k_cache = k_cache;
  f.v_cache = v_cache;
  f.err = err;
  switch (n_q / n_kv) {
    case 1: launch_fused_g<1>(f, ch, B, s); break;
    case 2: launch_fused_g<2>(f, ch, B, s); break;
    case 4: launch_fused_g<4>(f, ch, B, s); break;
    default: launch_fused_g<8>(f, ch, B, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_prompt_attention(const uint16_t* q, int S, int P, int ldq, int n_q, int n_kv,
                                   const uint16_t* k_cache, const uint16_t* v_cache, int max_pos,
                                   int pos_base, uint16_t* out, int ldo, hipStream_t s) {
  const int G = n_q / n_kv;
  PromptAttn a{q, ldq, k_cache, v_cache, n_kv, max_pos, P, pos_base, (P + kPQ / G - 1) / (kPQ / G),
               kLog2e / sqrtf((float)kHD), out, ldo};
  switch (G) {
    case 1: launch_prompt_g<1>(a, S, s); break;
    case 2: launch_prompt_g<2>(a, S, s); break;
    case 4: launch_prompt_g<4>(a, S, s); break;
    default: launch_prompt_g<8>(a, S, s); break;
  }
  return hipGetLastError();
}

}  // namespace m3
