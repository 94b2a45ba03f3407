#pragma once
// persist_kernel.h -- device side of the persistent frame (see persist.hip).
#include "frame_impl.h"
#include "persist_attn.h"
#include "cfg_impl.h"

namespace m3 {
namespace {

// Phase kinds.  A frame kernel is compiled for one body format FB (bf16 or
// int8-row, also the lm_head's) with the depth decoder in int8-g128: every
// variant it carries costs registers in all of them, so it carries only two:
// variant 0 = FB, 1 = int8-g128, the epilogue chosen at run time and the
// operand always staged in LDS (the frame is recorded only when it fits).
constexpr int kFeedbackVariant = -1;
// An attention phase (persist_attn.h), carried only by the kernels compiled
// with ATT (frames with decode attention), so the frames with the identity
// stub keep their registers.
constexpr int kAttnVariant = -2;
// A guided draw phase (the reference's draw: guidance over each song's row
// pair, top-k, Gumbel-argmax; cfg_impl.h), also carried only by the ATT
// kernels: it waits for every workgroup's flag of the logits GEMV before it,
// then workgroup s draws song s.
constexpr int kCfgVariant = -3;
constexpr int kCfgPersistThreads = kThreads;

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

// Phase clock (optional, m3_frame_persistent_clock): thread 0 of each
// workgroup writes the constant-rate real-time counter at the phase's entry
// (slot 0), when its operand is staged (slot 1) and at the phase's end
// (slot 2), to clk[(slot * nph + phase) * nwg + wg]; `at` points at slot 0's
// entry of the phase and workgroup, `stride` = nph * nwg.
__device__ __forceinline__ void clock_mark(uint64_t* at, size_t stride, int slot) {
  if (at && threadIdx.x == 0) at[slot * stride] = __builtin_amdgcn_s_memrealtime();
}

// GEMV phases wait inside their loads (tagged words): nothing to do before
// the weight stream but report whether the operand is plain and ready (phase
// 0 reads the launch's plain input).
struct TagWait {
  uint32_t eb;
  int i;
  uint32_t* er;
  uint64_t* clk;       // phase clock: slot 0 entry of this phase and workgroup (nullptr: off)
  size_t cstride;
  __device__ bool probe() const { return i == 0; }
  __device__ bool wait() const { return true; }
  // phase clock: this workgroup's operand is staged
  __device__ void staged() const { clock_mark(clk, cstride, 1); }
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
  gemv_run<FMT, NB, true, kGluRuntime, FMT == M3_I8G128 ? 4 : 8, true>(
      *(const Params*)&ph->p, smem, wg, nwg, wait);
}

// an attention phase of a kernel compiled with ATT: G = 1, 2, 4 query heads
// per KV head, chunks of 64 or 128 positions (false: not an attention phase)
template <bool ATT>
__device__ __forceinline__ bool run_attention(int variant, CPhasePtr ph, uint8_t* smem, int wg,
                                              int nwg, uint32_t ebase, int i, uint32_t* err,
                                              uint64_t* at, size_t cstride) {
  if constexpr (ATT) {
    if (variant != kAttnVariant) return false;
    const AttnArgs& a = *(const AttnArgs*)&ph->p;
    const int g = a.n_q / a.n_kv;
    auto staged = [&]() { clock_mark(at, cstride, 1); };
    if (a.ch == 64) {
      if (g == 1) attn_phase<1, 64>(a, smem, wg, nwg, ebase, i, err, staged);
      else if (g == 2) attn_phase<2, 64>(a, smem, wg, nwg, ebase, i, err, staged);
      else attn_phase<4, 64>(a, smem, wg, nwg, ebase, i, err, staged);
    } else {
      if (g == 1) attn_phase<1, 128>(a, smem, wg, nwg, ebase, i, err, staged);
      else if (g == 2) attn_phase<2, 128>(a, smem, wg, nwg, ebase, i, err, staged);
      else attn_phase<4, 128>(a, smem, wg, nwg, ebase, i, err, staged);
    }
    return true;
  } else {
    return false;
  }
}

// a guided draw phase of a kernel compiled with ATT (false: not one); false
// from wait: the launch gives up (a wait failed)
template <bool ATT>
__device__ __forceinline__ bool run_cfg(int variant, CPhasePtr ph, uint8_t* smem, int wg,
                                        const uint32_t* flags, int nwg, uint32_t ebase, int i,
                                        uint32_t* err, int* s_ok, uint64_t* at, size_t cstride,
                                        bool& ok) {
  if constexpr (ATT) {
    if (variant != kCfgVariant) return false;
    ok = wait_flags(flags, nwg, ebase + (uint32_t)i, err, s_ok);
    if (!ok) return true;
    clock_mark(at, cstride, 1);
    const CfgDesc& d = *(const CfgDesc*)&ph->p;
    if (wg < d.S) {
      int tx = threadIdx.x;              // (opaque: nothing derived is hoisted out of the loop)
      asm volatile("" : "+v"(tx));
      auto& sh = *reinterpret_cast<CfgShared<kCfgPersistThreads>*>(smem);
      const uint32_t ty = tag_of(i, ebase);
      if (d.V <= 2 * kCfgPersistThreads)
        cfg_song<2, kCfgPersistThreads, true>(d, wg, tx, sh, ty);
      else if (d.V <= 8 * kCfgPersistThreads)
        cfg_song<8, kCfgPersistThreads, true>(d, wg, tx, sh, ty);
      else
        cfg_song<36, kCfgPersistThreads, true>(d, wg, tx, sh, ty);
    }
    return true;
  } else {
    return false;
  }
}

template <int NB, int FB, bool CLK, bool ATT = false>
__global__ __launch_bounds__(kThreads) void frame_kernel(const Phase* ph, int nph, uint32_t* flags,
                                                         uint32_t* err, const uint32_t* seq,
                                                         FeedbackArgs fb, uint64_t* clk) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_ok;
  __shared__ int c_last[M3_MAX_B_FRAME];
  const int wg = blockIdx.x, nwg = gridDim.x;
  // a launch on a state whose error word is raised computes nothing: the
  // state must be recorded again (persistent_create) first
  if (__builtin_amdgcn_readfirstlane(ld4<true>(err, 0)) != 0u) return;
  // epochs of this launch: launch counter * 512 + phase + 1
  const uint32_t ebase = __builtin_amdgcn_readfirstlane(ld4<true>(seq, 0)) * kPhaseStride;
  const size_t cstride = (size_t)nph * nwg;
  for (int i = 0; i < nph; ++i) {
    const int variant = __builtin_amdgcn_readfirstlane(ph[i].variant);
    uint64_t* at = CLK ? clk + (size_t)i * nwg + wg : nullptr;   // (CLK: clk is set)
    clock_mark(at, cstride, 0);
    if (variant == kFeedbackVariant) {
      if (!wait_flags(flags, nwg, ebase + (uint32_t)i, err, &s_ok)) return;
      clock_mark(at, cstride, 1);
      feedback_run<true>(fb, wg, nwg, c_last, ebase);
    } else if (run_attention<ATT>(variant, (CPhasePtr)(ph + i), smem, wg, nwg, ebase, i, err, at, cstride)) {
    } else if (bool ok = true; run_cfg<ATT>(variant, (CPhasePtr)(ph + i), smem, wg, flags, nwg, ebase, i,
                                            err, &s_ok, at, cstride, ok)) {
      if (!ok) return;
    } else {
      TagWait wait{ebase, i, err, at, cstride};
      const CPhasePtr cp = (CPhasePtr)(ph + i);
      if (variant == 0)
        run_variant<FB, NB>(cp, smem, wg, nwg, wait);
      else
        run_variant<M3_I8G128, NB>(cp, smem, wg, nwg, wait);
    }
    if (__builtin_amdgcn_readfirstlane(ph[i].signal)) signal_epoch(flags, wg, ebase + (uint32_t)i + 1u);
    clock_mark(at, cstride, 2);
  }
}

}  // namespace
}  // namespace m3
