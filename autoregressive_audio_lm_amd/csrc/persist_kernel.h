#pragma once
// persist_kernel.h -- device side of the persistent frame (see persist.hip).
#include "frame_impl.h"

namespace m3 {
namespace {

constexpr long kSpinLimit = 1L << 21;        // polls (each a memory round trip) before giving up

// Phase kinds.  A frame kernel is compiled for one body format FB (bf16 or
// int8-row, also the lm_head's) with the depth decoder in int8-g128: every
// variant it carries costs registers in all of them, so it carries only
// these.  variant = class * 4 + arm; class 0 = FB, 1 = int8-g128; arm 0 =
// operand staged in LDS, 1 = the same with the SwiGLU epilogue, 2 = operand
// read from global memory (only compiled for 16-row tiles: below 5 rows every
// operand of the frame fits LDS).
constexpr int kArmLds = 0, kArmGlu = 1, kArmGlobal = 2;
constexpr int kFeedbackVariant = -1;

struct Phase {
  Params p;
  int variant;
  int pad[3];
};

template <int NB>
constexpr bool global_arm(int) { return NB >= 16; }

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

// The producer of phase i's operand is phase i-1 (all workgroups).  wait():
// wave 0 polls until done, or until the spin limit passed or another
// workgroup raised the error word.
struct PhaseWait {
  const uint32_t* flags;
  uint32_t* err;
  uint32_t target;
  int nwg;
  bool first;          // phase 0: the operand was written before the launch
  int* s_ok;
  bool* ok;

  // Looking costs a round trip before the weight stream starts, and most
  // workgroups find the producer still running: report "not ready" without
  // looking (except for phase 0) so that two batches stream during the wait.
  __device__ bool probe() { return first; }

  __device__ bool wait() {
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
    *ok = *s_ok != 0;
    return *ok;
  }
};

__device__ __forceinline__ void signal_epoch(uint32_t* flags, int wg, uint32_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);        // this thread's stores have completed
  __syncthreads();                      // ... and every other thread's
  if (threadIdx.x == 0) st4<true>(flags, (size_t)wg * 4, epoch);
}

typedef const __attribute__((address_space(4))) Phase* CPhasePtr;

// the phase's parameters are read from the (read-only) table in the
// constant address space, i.e. with scalar loads into wave-uniform registers
template <int FMT, int NB, bool LDS, bool GLU, class W>
__device__ __forceinline__ void run_variant(CPhasePtr ph, uint8_t* smem, int wg, int nwg, W& wait) {
  gemv_run<FMT, NB, (NB >= 16), LDS, GLU, (LDS && FMT == M3_I8G128) ? 4 : 8, true>(
      *(const Params*)&ph->p, smem, wg, nwg, wait);
}

template <int FMT, int NB, int CLS, class W>
__device__ __forceinline__ void run_class(CPhasePtr ph, uint8_t* smem, int wg, int nwg, int arm,
                                          W& wait) {
  if (arm == kArmLds) {
    run_variant<FMT, NB, true, false>(ph, smem, wg, nwg, wait);
  } else if (arm == kArmGlu) {
    run_variant<FMT, NB, true, true>(ph, smem, wg, nwg, wait);
  } else {
    if constexpr (global_arm<NB>(CLS)) run_variant<FMT, NB, false, false>(ph, smem, wg, nwg, wait);
  }
}

template <int NB, int FB>
__global__ __launch_bounds__(kThreads) void frame_kernel(const Phase* ph, int nph, uint32_t* flags,
                                                         uint32_t* err, const uint32_t* frame,
                                                         FeedbackArgs fb) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_ok;
  __shared__ int c_last[M3_MAX_B_FRAME];
  const int wg = blockIdx.x, nwg = gridDim.x;
  const uint32_t ebase = __builtin_amdgcn_readfirstlane(ld4<true>(frame, 0)) * kPhaseStride;
  for (int i = 0; i < nph; ++i) {
    const int variant = __builtin_amdgcn_readfirstlane(ph[i].variant);
    bool ok = true;
    PhaseWait wait{flags, err, ebase + (uint32_t)i, nwg, i == 0, &s_ok, &ok};
    if (variant == kFeedbackVariant) {
      if (wait.probe() || wait.wait()) feedback_run<true>(fb, wg, nwg, c_last);
    } else {
      const CPhasePtr cp = (CPhasePtr)(ph + i);
      if (variant < 4)
        run_class<FB, NB, 0>(cp, smem, wg, nwg, variant, wait);
      else
        run_class<M3_I8G128, NB, 1>(cp, smem, wg, nwg, variant - 4, wait);
    }
    if (!ok) return;
    signal_epoch(flags, wg, ebase + (uint32_t)i + 1u);
  }
}

}  // namespace
}  // namespace m3
