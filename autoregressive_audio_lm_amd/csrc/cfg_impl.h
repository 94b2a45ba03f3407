#pragma once
// cfg_impl.h -- device code of the reference's draw (guidance over a song's
// row pair, top-k, Gumbel-argmax), shared by its own kernel (sample.hip) and
// the persistent frame's draw phases (persist_kernel.h), so both draw the
// same ids.  Every floating-point step of the guided values is one IEEE fp32
// operation (no contraction); the search and the draw are exact.
#include "gemv_impl.h"

namespace m3 {

// ---- the reference's draw: guidance over row pairs, top-k, Gumbel-argmax ------
// DiffSynth-Studio MiniMax-Music3 stage 2: guided = u + 1.5 (c - u) from the
// conditional and unconditional rows of a song, top-k 50, multinomial
// sampling -- drawn here as Gumbel-argmax over the k survivors (the same law;
// diffusers issue #14486 item 3) on the plain draw's Philox counters with
// the song as the row word.
//
// One workgroup of NT threads per song (1024 in the draw's own kernel, 512
// in the persistent frame).  Thread t holds runs of W
// consecutive columns, run g at column g*NT*W + t*W (coalesced loads;
// column order = (run, thread, position)).  Guided values become
// order-preserving 32-bit keys in registers.  The k-th largest key T comes
// from a most-significant-first search, two bits per step: three
// block-wide counts #(key >= candidate) per step, taken with wave ballots
// and summed across waves through LDS and DPP row sums (no histograms, no
// atomics).  The search stops as soon as exactly k keys lie at or above the
// bound; once at most NT keys do, they are compacted into LDS in column
// order and the rest of the search runs on one key per thread.  Survivors
// are the keys above T plus the lowest-column keys equal to T, i.e. the k
// largest with ties to the lower column.
constexpr int kCfgMaxRuns = 9;       // runs of 4 columns per thread (V <= 32768 at 1024
                                     // threads, <= 18432 at 512)

template <int NT>
struct CfgShared {
  static constexpr int NW = NT / 64;  // waves (16 or 8: at most the 16 lanes of a DPP row)
  int4 red[2][NW];                    // block_sum3 slots (double-buffered)
  int wt[kCfgMaxRuns][NW];            // per-run wave totals for column-order ranks
  uint32_t ckey[NT];                  // compacted keys, in column order
  int ccol[NT];                       // ... and their columns
  Best wbest[NW];
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
// (zero past the last wave) and sums its row.  The slots are double-buffered
// by `par`, so one barrier per call suffices (a slot is rewritten two calls
// later, after every thread has passed the barrier in between).
template <int NT>
__device__ __forceinline__ int3 block_sum3(int a, int b, int c, CfgShared<NT>& sh, int& par,
                                           int tid) {
  constexpr int NW = CfgShared<NT>::NW;
  const int lane = tid & 63, wave = tid >> 6, lw = lane & 15;
  if (lane == 0) sh.red[par][wave] = make_int4(a, b, c, 0);
  __syncthreads();
  const int4 x = lw < NW ? sh.red[par][lw] : make_int4(0, 0, 0, 0);
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
template <int G, int W, int NT>
__device__ __forceinline__ int column_ranks(const bool (&f)[G][W], int (&start)[G], CfgShared<NT>& sh,
                                            int tid) {
  constexpr int NW = CfgShared<NT>::NW;
  const int lane = tid & 63, wave = tid >> 6, lw = lane & 15;
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
    const int x = lw < NW ? sh.wt[g][lw] : 0;
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
// record {0, j} per row (COH: a persistent launch's record, with tag `tag`).
template <bool COH>
__device__ __forceinline__ void cfg_write(const CfgDesc& d, int s, int j, uint32_t tag) {
  if (d.part) {
    const Best r = COH ? part_tag(Best{0.0f, j}, tag) : Best{0.0f, j};
    st_best<COH>(d.part, 2 * s, r);
    st_best<COH>(d.part, 2 * s + 1, r);
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
template <int G, int W, int NT>
__device__ __forceinline__ void search_step(const uint32_t (&k)[G][W], int kk, CfgSearch& st,
                                            CfgShared<NT>& sh, int& par, int tid) {
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
  const int3 r = block_sum3<NT>(n1, n2, n3, sh, par, tid);
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
template <int G, int W, int NT, bool COH>
__device__ __forceinline__ void cfg_finish(const CfgDesc& d, int s, const uint32_t (&k)[G][W],
                                           const int (&cols)[G][W], int kk, CfgSearch st,
                                           CfgShared<NT>& sh, int& par, int tid, uint32_t tag) {
  constexpr int NW = CfgShared<NT>::NW;
  const int lane = tid & 63, wave = tid >> 6, lw = lane & 15;
  while (!st.done && st.sh >= 0) search_step<G, W, NT>(k, kk, st, sh, par, tid);
  // survivors: keys above T, then keys equal to T in column order (all of
  // them when exactly k keys are >= T)
  int ngt = 0;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int q = 0; q < W; ++q) ngt += wave_count(k[g][q] > st.T);
  const int need = kk - block_sum3<NT>(ngt, 0, 0, sh, par, tid).x;
  const bool all_ties = st.nT == kk;
  bool tie[G][W];
  int start[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    start[g] = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) tie[g][q] = k[g][q] == st.T;
  }
  if (!all_ties) column_ranks<G, W, NT>(tie, start, sh, tid);
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
  // rows of 16 lanes, then the wave's four rows, then the waves
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
  bz = lw < NW ? sh.wbest[lw].z : -INFINITY;
  bj = lw < NW ? sh.wbest[lw].j : 0x7fffffff;
  best_row16(bz, bj);
  if (tid == 0) cfg_write<COH>(d, s, bj, tag);
}

// The draw of song s (rows 2 s, 2 s + 1) by the NT threads tid of one
// workgroup, E columns per thread (V <= NT E).  COH: inside a persistent
// launch (logits read with coherent loads, the winner records tagged `tag`).
template <int E, int NT, bool COH>
__device__ __forceinline__ void cfg_song(const CfgDesc& d, int s, int tid, CfgShared<NT>& sh,
                                         uint32_t tag) {
#pragma clang fp contract(off)
  constexpr int W = E < 4 ? E : 4;     // columns per run
  constexpr int G = E / W;             // runs per thread
  static_assert(G <= kCfgMaxRuns, "runs per thread");
  const float* c = d.logits + (size_t)(2 * s) * d.ldl;
  const float* u = c + d.ldl;
  // 1. guided values -> keys
  uint32_t k[G][W];
  int cols[G][W];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int j0 = g * (NT * W) + tid * W;
    float cv[W], uv[W];
    if (W == 4 && d.vec4 && j0 + 3 < d.V) {
      const uint4 a = ld16<COH>(c, (size_t)j0 * 4);
      const uint4 b = ld16<COH>(u, (size_t)j0 * 4);
      cv[0] = __uint_as_float(a.x); cv[1] = __uint_as_float(a.y);
      cv[2] = __uint_as_float(a.z); cv[3] = __uint_as_float(a.w);
      uv[0] = __uint_as_float(b.x); uv[1] = __uint_as_float(b.y);
      uv[2] = __uint_as_float(b.z); uv[3] = __uint_as_float(b.w);
    } else {
#pragma unroll
      for (int q = 0; q < W; ++q) {
        const bool in = j0 + q < d.V;
        cv[q] = in ? __uint_as_float(ld4<COH>(c, (size_t)(j0 + q) * 4)) : 0.0f;
        uv[q] = in ? __uint_as_float(ld4<COH>(u, (size_t)(j0 + q) * 4)) : 0.0f;
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
  const int n = block_sum3<NT>(nv, 0, 0, sh, par, tid).x;
  if (n == 0) {   // nothing to draw from: the first column's id
    if (tid == 0) cfg_write<COH>(d, s, 0, tag);
    return;
  }
  const int kk = d.top_k < n ? d.top_k : n;
  CfgSearch st{0u, 0, 30, false};
  if constexpr (E == 1) {
    cfg_finish<G, W, NT, COH>(d, s, k, cols, kk, st, sh, par, tid, tag);
  } else {
    // 3. search on every key until at most NT remain at or above the bound
    while (!st.done && st.sh >= 0 && !(st.T != 0u && st.nT <= NT))
      search_step<G, W, NT>(k, kk, st, sh, par, tid);
    if (st.done || st.sh < 0) {
      cfg_finish<G, W, NT, COH>(d, s, k, cols, kk, st, sh, par, tid, tag);
      return;
    }
    // 4. compact the keys >= T (column order kept) and finish on one per thread
    bool f[G][W];
    int start[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int q = 0; q < W; ++q) f[g][q] = k[g][q] >= st.T;
    column_ranks<G, W, NT>(f, start, sh, tid);
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
    cfg_finish<1, 1, NT, COH>(d, s, k1, c1, kk, st, sh, par, tid, tag);
  }
}


}  // namespace m3
