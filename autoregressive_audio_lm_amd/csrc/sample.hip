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
#include "m3_internal.h"
#include "m3_sampling.h"

#include <mutex>

#pragma clang fp contract(off)

namespace m3 {
namespace {

constexpr int kChunk = 1024;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gumbel_partial(SampleDesc d) {
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
  __shared__ Best sb[kThreads / 64];
  if (lane == 0) sb[wave] = Best{bz, bj};
  __syncthreads();
  if (tid == 0) {
    Best r = sb[0];
    for (int w = 1; w < kThreads / 64; ++w)
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
// DiffSynth-Studio MiniMax-Music3 stage 2: guided = u + 1.5 (c - u) from the
// conditional and unconditional rows of a song, top-k 50, multinomial
// sampling -- drawn here as Gumbel-argmax over the k survivors (the same law;
// diffusers issue #14486 item 3) on the plain draw's Philox counters with
// the song as the row word.
//
// One workgroup of 1024 threads per song.  Thread t holds runs of W
// consecutive columns, run g at column g*1024*W + t*W (coalesced loads;
// column order = (run, thread, position)).  Guided values become
// order-preserving 32-bit keys in registers.  The k-th largest key T comes
// from a most-significant-first search, two bits per step: three
// block-wide counts #(key >= candidate) per step, taken with wave ballots
// and summed across waves through LDS and DPP row sums (no histograms, no
// atomics).  The search stops as soon as exactly k keys lie at or above the
// bound; once at most 1024 keys do, they are compacted into LDS in column
// order and the rest of the search runs on one key per thread.  Survivors
// are the keys above T plus the lowest-column keys equal to T, i.e. the k
// largest with ties to the lower column.
constexpr int kCfgThreads = 1024;
constexpr int kCfgWaves = kCfgThreads / 64;
constexpr int kCfgMaxRuns = 8;       // runs of 4 columns per thread (V <= 32768)

struct CfgShared {
  int4 red[2][kCfgWaves];            // block_sum3 slots (double-buffered)
  int wt[kCfgMaxRuns][kCfgWaves];    // per-run wave totals for column-order ranks
  uint32_t ckey[kCfgThreads];        // compacted keys, in column order
  int ccol[kCfgThreads];             // ... and their columns
  Best wbest[kCfgWaves];
};

// order-preserving map of a non-NaN fp32 to uint32, -0 taken as +0; key 0
// never arises from a value, so it marks columns that take no part
__device__ __forceinline__ uint32_t cfg_key(float g) {
  const uint32_t b = __float_as_uint(g + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float cfg_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Sum over the 16 lanes of each DPP row, left in every lane of the row:
// quad exchanges 1 and 2, then half-row and row mirrors.
__device__ __forceinline__ int row_sum16(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);   // row_mirror
  return v;
}

// The best (z, j) of each DPP row, in every lane of the row (same steps).
template <int CTRL>
__device__ __forceinline__ void best_dpp_step(float& z, int& j) {
  const float oz = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), CTRL, 0xF, 0xF, false));
  const int oj = __builtin_amdgcn_update_dpp(0, j, CTRL, 0xF, 0xF, false);
  if (above(oz, oj, z, j)) {
    z = oz;
    j = oj;
  }
}

__device__ __forceinline__ void best_row16(float& z, int& j) {
  best_dpp_step<0xB1>(z, j);
  best_dpp_step<0x4E>(z, j);
  best_dpp_step<0x141>(z, j);
  best_dpp_step<0x140>(z, j);
}

// Block-wide sums of three per-wave counts (each already uniform in its
// wave): one slot per wave in LDS, then every lane reads slot (lane % 16)
// and sums its row.  The slots are double-buffered by `par`, so one barrier
// per call suffices (a slot is rewritten two calls later, after every thread
// has passed the barrier in between).
__device__ __forceinline__ int3 block_sum3(int a, int b, int c, CfgShared& sh, int& par) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh.red[par][wave] = make_int4(a, b, c, 0);
  __syncthreads();
  const int4 x = sh.red[par][lane & (kCfgWaves - 1)];
  par ^= 1;
  return make_int3(row_sum16(x.x), row_sum16(x.y), row_sum16(x.z));
}

// number of lanes of the wave where p holds (a compare and a scalar popcount)
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// lanes below this one where p holds
__device__ __forceinline__ int lanes_below(bool p) {
  const unsigned long long m = __ballot(p);
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Column-order ranks of flagged elements held as G runs of W per thread
// (order: run, thread, position).  start[g] = rank of this thread's first
// flagged element of run g; returns the number flagged.
template <int G, int W>
__device__ __forceinline__ int column_ranks(const bool (&f)[G][W], int (&start)[G], CfgShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lw = lane & (kCfgWaves - 1);
  int below[G], wtot[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) cnt += f[g][q];
    below[g] = 0;
    wtot[g] = 0;
#pragma unroll
    for (int b = 0; (1 << b) <= W; ++b) {
      const bool p = (cnt >> b) & 1;
      below[g] += lanes_below(p) << b;
      wtot[g] += wave_count(p) << b;
    }
  }
  __syncthreads();                       // earlier readers of wt are done
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) sh.wt[g][wave] = wtot[g];
  }
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int x = sh.wt[g][lw];
    const int all = row_sum16(x);
    start[g] = base + row_sum16(lw < wave ? x : 0) + below[g];
    base += all;
  }
  return base;
}

// absolute id of column j (an id list, the end token in column 0, or index_base + j)
__device__ __forceinline__ int32_t cfg_id(const CfgDesc& d, int j) {
  if (d.ids) return d.ids[j];
  return (d.end_id >= 0 && j == 0) ? d.end_id : d.index_base + j;
}

// The song's draw (column j) to both of its rows: the absolute id, or, for the
// frame's consumers (the gather prologue, the frame end), a one-entry winner
// record {0, j} per row.
__device__ __forceinline__ void cfg_write(const CfgDesc& d, int s, int j) {
  if (d.part) {
    d.part[2 * s] = Best{0.0f, j};
    d.part[2 * s + 1] = Best{0.0f, j};
    return;
  }
  const int32_t id = cfg_id(d, j);
  d.out[(size_t)(2 * s) * d.out_stride] = id;
  d.out[(size_t)(2 * s + 1) * d.out_stride] = id;
}

// Search state shared by both phases of the kernel.
struct CfgSearch {
  uint32_t T;   // lower bound of the k-th largest key
  int nT;       // #(key >= T), valid once T > 0
  int sh;       // next bit pair to decide
  bool done;    // exactly k keys >= T
};

// One two-bit search step over G x W keys per thread.
template <int G, int W>
__device__ __forceinline__ void search_step(const uint32_t (&k)[G][W], int kk, CfgSearch& st,
                                            CfgShared& sh, int& par) {
  const uint32_t c1 = st.T | (1u << st.sh), c2 = st.T | (2u << st.sh), c3 = st.T | (3u << st.sh);
  int n1 = 0, n2 = 0, n3 = 0;   // per wave
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int q = 0; q < W; ++q) {
      n1 += wave_count(k[g][q] >= c1);
      n2 += wave_count(k[g][q] >= c2);
      n3 += wave_count(k[g][q] >= c3);
    }
  }
  const int3 r = block_sum3(n1, n2, n3, sh, par);
  if (r.z >= kk) {
    st.T = c3;
    st.nT = r.z;
  } else if (r.y >= kk) {
    st.T = c2;
    st.nT = r.y;
  } else if (r.x >= kk) {
    st.T = c1;
    st.nT = r.x;
  }
  st.sh -= 2;
  st.done = st.T != 0u && st.nT == kk;
}

// Finish the search on G x W keys per thread (columns in cols), pick the
// survivors, draw, and write the song's two outputs.
template <int G, int W>
__device__ __forceinline__ void cfg_finish(const CfgDesc& d, int s, const uint32_t (&k)[G][W],
                                           const int (&cols)[G][W], int kk, CfgSearch st,
                                           CfgShared& sh, int& par) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lw = lane & (kCfgWaves - 1);
  while (!st.done && st.sh >= 0) search_step<G, W>(k, kk, st, sh, par);
  // survivors: keys above T, then keys equal to T in column order (all of
  // them when exactly k keys are >= T)
  int ngt = 0;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int q = 0; q < W; ++q) ngt += wave_count(k[g][q] > st.T);
  const int need = kk - block_sum3(ngt, 0, 0, sh, par).x;
  const bool all_ties = st.nT == kk;
  bool tie[G][W];
  int start[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    start[g] = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) tie[g][q] = k[g][q] == st.T;
  }
  if (!all_ties) column_ranks<G, W>(tie, start, sh);
  const uint32_t frame = d.frame_dev ? *d.frame_dev : d.frame;
  const float invT = inv_temperature(d.temperature);
  float bz = -INFINITY;
  int bj = 0x7fffffff;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int rank = start[g];
#pragma unroll
    for (int q = 0; q < W; ++q) {
      bool keep = k[g][q] > st.T;
      if (tie[g][q]) {
        keep = all_ties || rank < need;
        ++rank;
      }
      if (keep) {
        const int j = cols[g][q];
        const int32_t id = cfg_id(d, j);
        const float gn = d.noise ? d.noise[(size_t)s * d.V + j]
                                 : gumbel_noise(d.seed, (uint32_t)s, frame, d.draw, (uint32_t)id);
        const float z = gumbel_z(cfg_value(k[g][q]), invT, gn);
        if (above(z, j, bz, bj)) {
          bz = z;
          bj = j;
        }
      }
    }
  }
  // rows of 16 lanes, then the wave's four rows, then the 16 waves
  best_row16(bz, bj);
  {
    float mz = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bz)));
    int mj = __builtin_amdgcn_readfirstlane(bj);
    const float z1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bz), 16));
    const float z2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bz), 32));
    const float z3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bz), 48));
    const int j1 = __builtin_amdgcn_readlane(bj, 16);
    const int j2 = __builtin_amdgcn_readlane(bj, 32);
    const int j3 = __builtin_amdgcn_readlane(bj, 48);
    if (above(z1, j1, mz, mj)) { mz = z1; mj = j1; }
    if (above(z2, j2, mz, mj)) { mz = z2; mj = j2; }
    if (above(z3, j3, mz, mj)) { mz = z3; mj = j3; }
    bz = mz;
    bj = mj;
  }
  if (lane == 0) sh.wbest[wave] = Best{bz, bj};
  __syncthreads();
  bz = sh.wbest[lw].z;
  bj = sh.wbest[lw].j;
  best_row16(bz, bj);
  if (tid == 0) cfg_write(d, s, bj);
}

template <int E>
__global__ __launch_bounds__(kCfgThreads) void cfg_topk_kernel(CfgDesc d) {
  constexpr int W = E < 4 ? E : 4;     // columns per run
  constexpr int G = E / W;             // runs per thread
  __shared__ CfgShared sh;
  const int s = blockIdx.x, tid = threadIdx.x;
  const float* c = d.logits + (size_t)(2 * s) * d.ldl;
  const float* u = c + d.ldl;
  // 1. guided values -> keys
  uint32_t k[G][W];
  int cols[G][W];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int j0 = g * (kCfgThreads * W) + tid * W;
    float cv[W], uv[W];
    if (W == 4 && d.vec4 && j0 + 3 < d.V) {
      const float4 a = *reinterpret_cast<const float4*>(c + j0);
      const float4 b = *reinterpret_cast<const float4*>(u + j0);
      cv[0] = a.x; cv[1] = a.y; cv[2] = a.z; cv[3] = a.w;
      uv[0] = b.x; uv[1] = b.y; uv[2] = b.z; uv[3] = b.w;
    } else {
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const bool in = j0 + q < d.V;
        cv[q] = in ? c[j0 + q] : 0.0f;
        uv[q] = in ? u[j0 + q] : 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < W; ++q) {
      const int j = j0 + q;
      cols[g][q] = j;
      uint32_t key = 0u;
      if (j < d.V) {
        const int32_t id = cfg_id(d, j);
        if (!(d.valid_lo < d.valid_hi && (id < d.valid_lo || id >= d.valid_hi)) || id == d.end_id) {
          const float dl = cv[q] - uv[q];
          const float sd = d.scale * dl;
          const float gv = uv[q] + sd;
          if (gv == gv) key = cfg_key(gv);
        }
      }
      k[g][q] = key;
    }
  }
  // 2. candidates
  int nv = 0;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int q = 0; q < W; ++q) nv += wave_count(k[g][q] != 0u);
  int par = 0;
  const int n = block_sum3(nv, 0, 0, sh, par).x;
  if (n == 0) {   // nothing to draw from: the first column's id
    if (tid == 0) cfg_write(d, s, 0);
    return;
  }
  const int kk = d.top_k < n ? d.top_k : n;
  CfgSearch st{0u, 0, 30, false};
  if constexpr (E == 1) {
    cfg_finish<G, W>(d, s, k, cols, kk, st, sh, par);
  } else {
    // 3. search on every key until at most 1024 remain at or above the bound
    while (!st.done && st.sh >= 0 && !(st.T != 0u && st.nT <= kCfgThreads))
      search_step<G, W>(k, kk, st, sh, par);
    if (st.done || st.sh < 0) {
      cfg_finish<G, W>(d, s, k, cols, kk, st, sh, par);
      return;
    }
    // 4. compact the keys >= T (column order kept) and finish on one per thread
    bool f[G][W];
    int start[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int q = 0; q < W; ++q) f[g][q] = k[g][q] >= st.T;
    column_ranks<G, W>(f, start, sh);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int r = start[g];
#pragma unroll
      for (int q = 0; q < W; ++q) {
        if (f[g][q]) {
          sh.ckey[r] = k[g][q];
          sh.ccol[r] = cols[g][q];
          ++r;
        }
      }
    }
    __syncthreads();
    uint32_t k1[1][1];
    int c1[1][1];
    k1[0][0] = tid < st.nT ? sh.ckey[tid] : 0u;
    c1[0][0] = tid < st.nT ? sh.ccol[tid] : 0;
    cfg_finish<1, 1>(d, s, k1, c1, kk, st, sh, par);
  }
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
  hipLaunchKernelGGL(gumbel_partial, dim3(nchunk, d.B), dim3(kThreads), 0, s, d);
  hipLaunchKernelGGL(gumbel_final, dim3(d.B), dim3(64), 0, s, d, nchunk);
  return hipGetLastError();
}

}  // namespace m3
