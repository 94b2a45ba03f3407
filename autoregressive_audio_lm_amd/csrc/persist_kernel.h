#pragma once
// persist_kernel.h -- device side of the persistent frame (see persist.hip).
#include "frame_impl.h"

namespace m3 {
namespace {

// Phase kinds.  A frame kernel is compiled for one body format FB (bf16 or
// int8-row, also the lm_head's) with the depth decoder in int8-g128: every
// variant it carries costs registers in all of them, so it carries only two:
// variant 0 = FB, 1 = int8-g128, the epilogue chosen at run time and the
// operand always staged in LDS (the frame is recorded only when it fits).
constexpr int kFeedbackVariant = -1;

struct Phase {
  Params p;
  int variant;
  int signal;          // publish completion through the flags (the frame end waits for it)
  int pad[2];
};

// has every workgroup's flag reached `target`?  (wave 0; one coherent load per lane)
__device__ __forceinline__ bool flags_reached(const uint32_t* flags, int nwg, uint32_t target) {
  const int lane = threadIdx.x & 63;
  bool done = true;
  for (int w = lane * 4; w < nwg; w += 256) {
    const uint4 f = ld16<true>(flags, (size_t)w * 4);
    done = done && (int)(f.x - target) >= 0 && (int)(f.y - target) >= 0 &&
           (int)(f.z - target) >= 0 && (int)(f.w - target) >= 0;
  }
  return __all(done);
}

// GEMV phases wait inside their loads (tagged words): nothing to do before
// the weight stream but report whether the operand is plain and ready (phase
// 0 reads the launch's plain input).
struct TagWait {
  uint32_t eb;
  int i;
  uint32_t* er;
  __device__ bool probe() const { return i == 0; }
  __device__ bool wait() const { return true; }
  __device__ uint32_t ebase() const { return eb; }
  __device__ int phase() const { return i; }
  __device__ uint32_t* err() const { return er; }
};

// The frame end waits for every workgroup's flag of the phase before it:
// wave 0 polls until done, the spin limit passed or the error word is raised.
__device__ bool wait_flags(const uint32_t* flags, int nwg, uint32_t target, uint32_t* err, int* s_ok) {
  if (threadIdx.x < 64) {
    int good = 1;
    long spins = 0;
    while (!flags_reached(flags, nwg, target)) {
      if ((++spins & 63) == 0 && (spins > kSpinLimit || ld4<true>(err, 0) != 0u)) {
        good = 0;
        break;
      }
    }
    if (threadIdx.x == 0) {
      *s_ok = good;
      if (!good) st4<true>(err, 0, 1u);
    }
  }
  __syncthreads();
  return *s_ok != 0;
}

__device__ __forceinline__ void signal_epoch(uint32_t* flags, int wg, uint32_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);        // this thread's stores have completed
  __syncthreads();                      // ... and every other thread's
  if (threadIdx.x == 0) st4<true>(flags, (size_t)wg * 4, epoch);
}

typedef const __attribute__((address_space(4))) Phase* CPhasePtr;

// the phase's parameters are read from the (read-only) table in the
// constant address space, i.e. with scalar loads into wave-uniform registers
template <int FMT, int NB, class W>
__device__ __forceinline__ void run_variant(CPhasePtr ph, uint8_t* smem, int wg, int nwg, W& wait) {
  gemv_run<FMT, NB, (NB >= 16), true, kGluRuntime, FMT == M3_I8G128 ? 4 : 8, true>(
      *(const Params*)&ph->p, smem, wg, nwg, wait);
}

template <int NB, int FB>
__global__ __launch_bounds__(kThreads) void frame_kernel(const Phase* ph, int nph, uint32_t* flags,
                                                         uint32_t* err, const uint32_t* seq,
                                                         FeedbackArgs fb) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_ok;
  __shared__ int c_last[M3_MAX_B_FRAME];
  const int wg = blockIdx.x, nwg = gridDim.x;
  // epochs of this launch: launch counter * 512 + phase + 1
  const uint32_t ebase = __builtin_amdgcn_readfirstlane(ld4<true>(seq, 0)) * kPhaseStride;
  for (int i = 0; i < nph; ++i) {
    const int variant = __builtin_amdgcn_readfirstlane(ph[i].variant);
    if (variant == kFeedbackVariant) {
      if (!wait_flags(flags, nwg, ebase + (uint32_t)i, err, &s_ok)) return;
      feedback_run<true>(fb, wg, nwg, c_last, ebase);
    } else {
      TagWait wait{ebase, i, err};
      const CPhasePtr cp = (CPhasePtr)(ph + i);
      if (variant == 0)
        run_variant<FB, NB>(cp, smem, wg, nwg, wait);
      else
        run_variant<M3_I8G128, NB>(cp, smem, wg, nwg, wait);
    }
    if (__builtin_amdgcn_readfirstlane(ph[i].signal)) signal_epoch(flags, wg, ebase + (uint32_t)i + 1u);
  }
}

}  // namespace
}  // namespace m3
