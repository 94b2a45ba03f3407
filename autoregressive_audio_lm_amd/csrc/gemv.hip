// gemv.hip -- one RMSNorm-fused GEMV per launch (the C-ABI GEMV entry points
// and the graph-replayed frame).  The device code lives in gemv_impl.h.
#include "gemv_impl.h"

#include <algorithm>

namespace m3 {
namespace {

template <int FMT, int NB, bool LDS, bool GLU, int KU>
hipError_t configure_one() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemv_kernel<FMT, NB, LDS, GLU, KU>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  return status;
}

template <int FMT, int NB, bool LDS, bool GLU, int KU>
hipError_t launch_ku(const Params& p, int grid, size_t smem, hipStream_t s) {
  const hipError_t e = configure_one<FMT, NB, LDS, GLU, KU>();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemv_kernel<FMT, NB, LDS, GLU, KU>), dim3(grid), dim3(kThreads), smem,
                     s, p);
  return hipGetLastError();
}

template <int FMT, int NB, bool LDS, bool GLU>
hipError_t launch_epi(const Params& p, int grid, size_t smem, hipStream_t s) {
  return launch_ku<FMT, NB, LDS, GLU, (LDS && FMT == M3_I8G128) ? 4 : 8>(p, grid, smem, s);
}

template <int FMT, int NB, bool LDS>
hipError_t launch_one(const Params& p, int grid, size_t smem, hipStream_t s) {
  if (p.epi == M3_EPI_SWIGLU) return launch_epi<FMT, NB, LDS, true>(p, grid, smem, s);
  return launch_epi<FMT, NB, LDS, false>(p, grid, smem, s);
}

template <int FMT, bool LDS>
hipError_t dispatch_b(const Params& p, int grid, size_t smem, hipStream_t s) {
  const int B = p.B;
  if (B <= 16) return launch_one<FMT, 16, LDS>(p, grid, smem, s);
  if (B <= 32) return launch_one<FMT, 32, LDS>(p, grid, smem, s);
  if (B <= 48) return launch_one<FMT, 48, LDS>(p, grid, smem, s);
  return launch_one<FMT, 64, LDS>(p, grid, smem, s);
}

template <int FMT, bool LDS, bool GLU, int KU>
hipError_t configure_ku() {
  const hipError_t es[] = {
      configure_one<FMT, 16, LDS, GLU, KU>(),  configure_one<FMT, 32, LDS, GLU, KU>(),
      configure_one<FMT, 48, LDS, GLU, KU>(),  configure_one<FMT, 64, LDS, GLU, KU>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

template <int FMT, bool LDS, bool GLU>
hipError_t configure_epi() {
  return configure_ku<FMT, LDS, GLU, (LDS && FMT == M3_I8G128) ? 4 : 8>();
}

template <int FMT, bool LDS>
hipError_t configure_fmt() {
  const hipError_t es[] = {configure_epi<FMT, LDS, false>(), configure_epi<FMT, LDS, true>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Split along K, for a GEMV without a fused norm whose B-row operand does not
// fit LDS (the body's down projection, K = 12288, from B = 7 on): the
// one-launch kernel then reads its operand from memory beside the weights,
// every workgroup the whole B x K of it, as many bytes as the weights of its
// row block.  Here workgroup (g, q) takes the K-slices of waves q W .. q W +
// W - 1 of the one-launch kernel for the R = 8 / W row blocks of group g:
// its operand window (K / R columns) is staged once in LDS and read by all of
// them.  Wave v streams row block g R + v / W over the K-slice of wave q W +
// v % W -- the same tiles in the same order, in the same batches, as that
// wave of the one-launch kernel -- and leaves its accumulators in the
// caller's fp32 partials; the last workgroup of the group to finish sums the
// 8 slices of each of its row blocks in wave order and runs the epilogue
// (finish_block), so every output is bit-identical to the one-launch kernel's.
// ---------------------------------------------------------------------------
constexpr int kSplitW = 2;                    // wave K-slices per workgroup
constexpr int kSplitR = kWaves / kSplitW;     // row blocks per group = K parts
constexpr int kSplitMaxLds = 128 * 1024;      // the operand window's LDS at most

// [first, last) tile of wave w's K-slice
__host__ __device__ inline int split_tlo(int T, int TPU, int w) {
  return ((T / TPU) * w / kWaves) * TPU;
}

template <int FMT, int KU>
__global__ __launch_bounds__(kThreads) void gemv_split_kernel(Params p, float* part, uint32_t* cnt) {
  constexpr int NB = 16;
  constexpr int TPU = FMT == M3_I8G128 ? 2 : 1;
  constexpr int TK = FMT == M3_BF16 ? 32 : 64;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_last;
  uint16_t* act = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int v = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x / kSplitR, q = blockIdx.x % kSplitR;
  const int rb = g * kSplitR + v / kSplitW;              // this wave's row block
  const int wave = q * kSplitW + v % kSplitW;            // whose K-slice it takes
  const int t_lo = split_tlo(p.T, TPU, wave);
  const int ntw = split_tlo(p.T, TPU, wave + 1) - t_lo;
  const int units = p.T / TPU;
  const int nbat = ((units + kWaves - 1) / kWaves * TPU + KU - 1) / KU;   // as the one-launch kernel
  const int w_lo = split_tlo(p.T, TPU, q * kSplitW) * TK;                 // window start (elements)
  const int wlen = split_tlo(p.T, TPU, q * kSplitW + kSplitW) * TK - w_lo;
  const int stride = p.lds_stride;                       // longest window + zero tile + 8
  const int zoff = stride - 8 - TK;                      // the zero tile
  const bool live = rb < p.nblocks;
  Tags tg;
  tg.x = tg.res = tg.u = tg.part = tg.y = kPlain;
  tg.err = nullptr;

  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(p.w, (uint32_t)((size_t)p.nblocks * p.bbytes));
  const uint32_t vlane = (uint32_t)lane * 16u, vlane_oob = vlane + kOob;
  const int G = p.K / 128;
  auto load = [&](uint4* dst, float* sc, int j) {
    const bool on = live && j < nbat;
    const uint32_t base = (uint32_t)((size_t)(live ? rb : 0) * p.bbytes) + (uint32_t)t_lo * kTileBytes;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int tt = j * KU + i;
      const bool real = on && tt < ntw;
      dst[i] = ldw<FMT == M3_I8G128 ? 0 : 2>(wr, real ? vlane : vlane_oob,
                                             real ? base + (uint32_t)tt * kTileBytes : 0u);
    }
    if constexpr (FMT == M3_I8G128) {
      const uint32_t g0 = (uint32_t)(t_lo + j * KU) >> 1;
      const uint32_t sbase = (uint32_t)((size_t)(live ? rb : 0) * p.bbytes) +
                             (uint32_t)p.T * kTileBytes + g0 * 4u;
      const uint32_t vrow = (uint32_t)(lane & 15) * (uint32_t)G * 4u;
#pragma unroll
      for (int k = 0; k < KU / 2; ++k) {
        const bool real = on && j * KU + 2 * k < ntw;
        sc[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            wr, real ? vrow : vrow + kOob, real ? sbase + 4u * k : 0u, 0));
      }
    }
  };
  Accum<FMT, NB> A;
  A.reset();
  auto compute = [&](const uint4* src, const float* scv, int j) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int tt = j * KU + i;
      const bool real = tt < ntw;
      A.template tile<true, false>(p, act, src[i], real ? (t_lo + tt) * TK - w_lo : zoff, tg);
      if (FMT == M3_I8G128 && (i & 1)) A.group_end(real ? scv[i >> 1] : 0.f);
    }
  };

  // the operand window of every row (zeros past K and past this window), its
  // first requests ahead of the first weight batch (loads retire in order)
  constexpr int U = 8;
  const int cpr = (stride - 8) >> 3;
  const int total = p.B * cpr;
  uint4 xv[U];
  auto fetch = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = base + u * kThreads + tid;
      const int b = it / cpr, k = (it - b * cpr) * 8;
      const bool in = it < total && k < wlen && w_lo + k < p.K;
      xv[u] = in ? load_x8<false>(p, b, w_lo + k, tg) : make_uint4(0, 0, 0, 0);
    }
  };
  auto put = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = base + u * kThreads + tid;
      if (it < total) {
        const int b = it / cpr, k = (it - b * cpr) * 8;
        *reinterpret_cast<uint4*>(act + (size_t)b * stride + k) = xv[u];
      }
    }
  };
  uint4 bufA[KU], bufB[KU];
  float scA[KU / 2], scB[KU / 2];
  fetch(0);
  load(bufA, scA, 0);
  put(0);
  for (int base = U * kThreads; base < total; base += U * kThreads) {
    fetch(base);
    put(base);
  }
  __syncthreads();
  load(bufB, scB, 1);
  __builtin_amdgcn_sched_barrier(0);
  for (int j = 0; j < nbat; j += 2) {
    compute(bufA, scA, j);
    load(bufA, scA, j + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 >= nbat) break;
    compute(bufB, scB, j + 1);
    load(bufB, scB, j + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  // this wave's slice sums: the [wave][row][16] record of its row block,
  // written through to memory (system-coherent stores: the workgroup that
  // combines them may sit on another XCD, whose L2 is not coherent with this
  // one's), completed before the group's counter is advanced
  constexpr int kRec = kWaves * NB * 16;                 // floats per row block
  if (live) {
    float* dst = part + (size_t)rb * kRec;
#pragma unroll
    for (int bt = 0; bt < NB / 16; ++bt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        st4<true>(dst, (size_t)((wave * NB + bt * 16 + 4 * (lane >> 4) + qq) * 16 + (lane & 15)) * 4,
                  __float_as_uint(A.acc[bt][qq]));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(cnt + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
             (uint32_t)(kSplitR - 1);
  __syncthreads();
  if (!s_last) return;
  // the last of the group: every record of its row blocks, read past the
  // caches into LDS (the operand window is no longer read), then the
  // one-launch kernel's cross-wave sum and epilogue for each
  float* red = reinterpret_cast<float*>(smem);
  const int nrb = min(kSplitR, p.nblocks - g * kSplitR);
  const float* src = part + (size_t)g * kSplitR * kRec;
  for (int i = tid; i < nrb * kRec / 4; i += kThreads) {
    const uint4 w4 = ld16<true>(src, (size_t)i * 16);
    *reinterpret_cast<uint4*>(red + 4 * i) = w4;
  }
  __syncthreads();
  for (int r = 0; r < nrb; ++r) {
    const int rbx = g * kSplitR + r;
    finish_block<FMT, NB, 0, false>(p, p.w + (size_t)rbx * p.bbytes, rbx, red + (size_t)r * kRec, tg);
  }
  if (tid == 0) st4<true>(cnt, (size_t)g * 4, 0u);       // ready for the next launch
}

template <int FMT, int KU>
hipError_t configure_split() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemv_split_kernel<FMT, KU>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kSplitMaxLds);
  return status;
}

// the split's LDS row stride (elements) for (fmt, K): the longest window,
// the zero tile and 8 of bank skew
int split_stride(int fmt, int K) {
  const int T = n_tiles(fmt, K), TPU = fmt == M3_I8G128 ? 2 : 1, TK = tile_k(fmt);
  int wmax = 0;
  for (int q = 0; q < kSplitR; ++q) {
    const int len = split_tlo(T, TPU, q * kSplitW + kSplitW) - split_tlo(T, TPU, q * kSplitW);
    wmax = len > wmax ? len : wmax;
  }
  return wmax * TK + TK + 8;
}

// LDS of the operand window, and of a group's records in the combine
size_t split_smem_bytes(int B, int stride) { return (size_t)B * stride * 2; }
size_t split_rec_bytes() { return (size_t)kSplitR * kWaves * 16 * 16 * sizeof(float); }

// the split runs when the caller gave its workspace, the GEMV has no fused
// norm, sampling, gather or SwiGLU, B <= 16, and the operand does not fit LDS
// whole but its window does.  (Where the whole operand fits, the split lost:
// O at B = 6 and 16 split made the graph frame 4.85 against 4.62 ms and 5.30
// against 5.24 ms, its combine's tail costing more than the staging saved.)
bool split_applies(const GemvDesc& d, bool lds) {
  if (lds || !d.kpart || !d.kcnt || d.gamma || d.sample || d.gather) return false;
  if (d.epi == M3_EPI_SWIGLU || d.B > 16 || n_blocks(d.N) > d.kpart_blocks) return false;
  return split_smem_bytes(d.B, split_stride(d.fmt, d.K)) <= (size_t)kSplitMaxLds;
}

template <int FMT, int KU>
hipError_t launch_split(Params p, const GemvDesc& d, hipStream_t s) {
  const hipError_t e = configure_split<FMT, KU>();
  if (e != hipSuccess) return e;
  p.lds_stride = split_stride(d.fmt, d.K);
  p.lds_rows = d.B;
  const int grid = (p.nblocks + kSplitR - 1) / kSplitR * kSplitR;
  const size_t smem = std::max(split_smem_bytes(d.B, p.lds_stride), split_rec_bytes());
  hipLaunchKernelGGL((gemv_split_kernel<FMT, KU>), dim3(grid), dim3(kThreads), smem, s, p, d.kpart,
                     d.kcnt);
  return hipGetLastError();
}

}  // namespace

size_t gemv_split_part_bytes(int nblocks) {
  return (size_t)nblocks * kWaves * 16 * 16 * sizeof(float);
}
size_t gemv_split_counters(int nblocks) { return (size_t)(nblocks + kSplitR - 1) / kSplitR; }

size_t gemv_smem_bytes(int fmt, int K, int B, bool has_gamma) {
  return smem_bytes_of(fmt, K, B, has_gamma);
}

hipError_t gemv_prepare() {
  const hipError_t es[] = {configure_fmt<M3_BF16, true>(),   configure_fmt<M3_BF16, false>(),
                           configure_fmt<M3_I8ROW, true>(),  configure_fmt<M3_I8ROW, false>(),
                           configure_fmt<M3_I8G128, true>(), configure_fmt<M3_I8G128, false>(),
                           configure_fmt<M3_FP8ROW, true>(), configure_fmt<M3_FP8ROW, false>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  const hipError_t ss[] = {configure_split<M3_BF16, 8>(), configure_split<M3_I8ROW, 8>(),
                           configure_split<M3_FP8ROW, 8>(), configure_split<M3_I8G128, 8>(),
                           configure_split<M3_I8G128, 4>()};
  for (hipError_t e : ss)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_gemv(const GemvDesc& d, hipStream_t s) {
  bool lds;
  int ku;      // fixed by the format (see ku_of); the instantiation below follows the same rule
  const Params p = make_params(d, &lds, &ku);
  if (d.gather && !lds) return hipErrorInvalidValue;   // the gather stages through LDS
  if (split_applies(d, lds)) {
    // (the batch size of the one-launch kernel it replaces: ku)
    switch (d.fmt) {
      case M3_BF16: return launch_split<M3_BF16, 8>(p, d, s);
      case M3_I8ROW: return launch_split<M3_I8ROW, 8>(p, d, s);
      case M3_FP8ROW: return launch_split<M3_FP8ROW, 8>(p, d, s);
      default:
        return ku == 4 ? launch_split<M3_I8G128, 4>(p, d, s) : launch_split<M3_I8G128, 8>(p, d, s);
    }
  }
  const size_t smem = smem_bytes_of(d.fmt, d.K, d.B, d.gamma != nullptr) +
                      (lds ? gamma_lds_bytes(d.fmt, d.gamma != nullptr, d.gather != nullptr, p.lds_rows,
                                             p.lds_stride, d.K, nb_of(d.B))
                           : 0);
  // resident workgroups per CU from LDS (8 waves each, at most 2 per CU)
  int per_cu = (int)((160 * 1024) / (smem + 1024));
  per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
  // with a fused norm every workgroup normalises the whole B x K operand:
  // one workgroup per CU does it once per CU.  (Measured on the graph frame,
  // preset A: B = 6 4.55 -> 4.17 ms, B = 16 5.15 -> 5.04 ms, B = 1 3.72 ->
  // 3.63 ms, B = 2 3.82 -> 3.74 ms.)
  if (d.gamma) per_cu = 1;
  int grid = 256 * per_cu;
  if (grid > p.nblocks) grid = p.nblocks;
  switch (d.fmt) {
    case M3_BF16:
      return lds ? dispatch_b<M3_BF16, true>(p, grid, smem, s)
                 : dispatch_b<M3_BF16, false>(p, grid, smem, s);
    case M3_I8ROW:
      return lds ? dispatch_b<M3_I8ROW, true>(p, grid, smem, s)
                 : dispatch_b<M3_I8ROW, false>(p, grid, smem, s);
    case M3_FP8ROW:
      return lds ? dispatch_b<M3_FP8ROW, true>(p, grid, smem, s)
                 : dispatch_b<M3_FP8ROW, false>(p, grid, smem, s);
    default:
      return lds ? dispatch_b<M3_I8G128, true>(p, grid, smem, s)
                 : dispatch_b<M3_I8G128, false>(p, grid, smem, s);
  }
}

}  // namespace m3
