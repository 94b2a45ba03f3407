#pragma once
// gemv_impl.h -- device code of the RMSNorm-fused skinny GEMV/GEMM over
// packed bf16 / int8-row / int8-group-128 weights for gfx950 (MI355X), shared
// by the one-GEMV-per-launch kernels (gemv.hip) and the persistent frame
// kernel (persist.hip).
//
// What is computed (TensorFold PR #987, precision list and "What it adds";
// DiffSynth-Studio MiniMax-Music3 model overview):
//   a = x                              (no norm)
//   a[b,k] = bf16(x[b,k] * r_b * g[k]) r_b = (mean_k x^2 + eps)^-1/2, fp32
//   y[b,n] = epi( sum_k W[n,k] a[b,k] ) with fp32 accumulation.
//
// Design (MI355X-first):
//  * The weights are the only large stream (the decode is bandwidth bound:
//    diffusers issue #14486 item 4 counts ~23 GB of weight reads per frame).
//    They are packed in 1 KB tiles (16 rows x 64 B) so that one 16-byte load
//    per lane of a wave64 fetches a whole tile contiguously.  Every weight
//    byte is read exactly once per call.
//  * A workgroup of 8 waves owns a block of 16 output rows; wave w owns a
//    fixed slice of K (a function of K only).  The reduction order of every
//    output therefore depends only on K -- never on N, B, the grid or where a
//    slice of rows starts -- so a sliced lm_head reproduces the full one bit
//    for bit, and row b never depends on the other rows.
//  * The activation block (after the fused RMSNorm) is staged once per
//    workgroup in LDS (row stride padded by 16 B against bank conflicts) and
//    re-used for every tile; workgroups loop over row blocks when there are
//    more blocks than resident workgroups.
//  * Every row count runs on v_mfma_f32_16x16x32_bf16 in tiles of 16
//    activation rows (A = 16 activation rows, B = the weight tile, exactly
//    the packed lane layout); rows past B repeat row B-1 and are not stored.
//  * int8 is dequantised to bf16 exactly (|q| <= 127 has 7 significant bits)
//    with one SDWA sign-extending convert per byte; scales are applied per row
//    (i8row) or per group of 128 along K (i8g128).
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct Params {
  const uint8_t* w;
  int N, K, Kp, T, nblocks;
  size_t bbytes;
  const uint16_t* x;
  int ldx, B;
  const float* gamma;
  float eps;
  int stub_group, stub_voff;
  void* y;
  int ldy, out_f32, epi;
  const uint16_t* res;
  int ldr;
  int lds_rows;        // activation rows staged in LDS (0: direct global reads)
  int lds_stride;      // LDS row stride in elements: Kp + one zero tile + 8 (bank skew)
  int has_sample, has_gather;
  SampleEpi smp;       // sampling epilogue (logits GEMVs)
  GatherPro gat;       // gather prologue (first GEMV of a depth step)
  // persistent launch only: the phase that produced each input (-1: a plain
  // bf16 buffer written before the launch) and whether outputs are tagged
  int px, pres, pu, ppart, ytag;
  int rot, follow;     // block order and workgroup offset (GemvDesc)
};

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// two fp32 -> packed bf16 pair with the hardware's round-to-nearest-even
// convert (v_cvt_pk_bf16_f32; one instruction for two values; finite values
// round exactly as f2bf, NaN stays NaN)
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf_pair(float lo, float hi) {
  const f32x2v_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v_t));
}

// ---------------------------------------------------------------------------
// RMSNorm (TensorFold PR #987 precision list: fp32 norms, bf16 operands).
// r comes from a float64 sum of squares (each square of a bf16 is exact in
// float64, and so is their sum over the ranges activations take, in any
// order) and is rounded once to fp32; each element is then
// bf16(fl32(fl32(x r) gamma)).  Every step is one IEEE operation, so the bf16
// rounding of each element is fixed by the steps and not by the order of a
// reduction: an operand element one ulp apart would shift every output of its
// row by W[n, k] ulp(a_k), enough to change the rounding of a few percent of
// them.
// ---------------------------------------------------------------------------
// one bf16 pair (x in the low and high halves of w) normalised with r and
// the gammas g0, g1 (two fp32 products each, one bf16 rounding)
__device__ __forceinline__ uint32_t norm_pair(uint32_t w, float r, float g0, float g1) {
  const float a0 = (__uint_as_float(w << 16) * r) * g0;
  const float a1 = (__uint_as_float(w & 0xffff0000u) * r) * g1;
  return f2bf_pair(a0, a1);
}

// sum of squares of a bf16 pair, added in float64 (each square is exact)
__device__ __forceinline__ double sumsq_pair(uint32_t w, double ss) {
  const double x0 = (double)__uint_as_float(w << 16), x1 = (double)__uint_as_float(w & 0xffff0000u);
  return fma(x1, x1, fma(x0, x0, ss));
}

// r = 1 / sqrt(ss / K + eps) in float64, rounded once to fp32: the hardware
// reciprocal square root refined by two Newton steps, each of which doubles
// its correct bits, so r is within a few float64 ulps before its fp32
// rounding (which it changes only when r lies that close to a tie between
// two fp32 values); a zero or infinite estimate (x infinite or zero, r = 0
// or infinity) is exact as it stands.
__device__ __forceinline__ float norm_r(double ss, int K, float eps) {
  const double x = ss / (double)K + (double)eps;
  double y = __builtin_amdgcn_rsq(x);
  if (y > 0.0 && y < __builtin_huge_val()) {
    const double h = 0.5 * x;
    y = y * fma(-h * y, y, 1.5);
    y = y * fma(-h * y, y, 1.5);
  }
  return (float)y;
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, a), acc, false);
}

// four int8 (one dword) -> two dwords of bf16 pairs (exact)
__device__ __forceinline__ void i8x4_to_bf16x4(uint32_t v, uint32_t& lo, uint32_t& hi) {
  float f0 = (float)(int8_t)(v & 0xffu);
  float f1 = (float)(int8_t)((v >> 8) & 0xffu);
  float f2 = (float)(int8_t)((v >> 16) & 0xffu);
  float f3 = (float)((int32_t)v >> 24);
  // the upper halves of two floats side by side: one byte permute per pair
  lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

__device__ __forceinline__ void i8x16_to_bf16(const uint4& q, uint32_t* o) {
  i8x4_to_bf16x4(q.x, o[0], o[1]);
  i8x4_to_bf16x4(q.y, o[2], o[3]);
  i8x4_to_bf16x4(q.z, o[4], o[5]);
  i8x4_to_bf16x4(q.w, o[6], o[7]);
}

// four fp8 (OCP E4M3) codes -> two dwords of bf16 pairs, exact: every E4M3
// value (subnormals included) is a bf16; the hardware pair convert with scale
// 1 does it in one instruction per pair
typedef __bf16 bf16x2p_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void f8x16_to_bf16(const uint4& q, uint32_t* o) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
  }
}

// one-byte codes of format FMT -> bf16 pairs
template <int FMT>
__device__ __forceinline__ void bytes16_to_bf16(const uint4& q, uint32_t* o) {
  if constexpr (FMT == M3_FP8ROW)
    f8x16_to_bf16(q, o);
  else
    i8x16_to_bf16(q, o);
}

// Sum over the wave, left in every lane, without LDS round trips: lane l
// and l^32, then l and l^16, with the permlane swaps (each adds the same two
// values in the same order in both lanes), then the 16 lanes of a row with
// DPP quad exchanges and half-row / row mirrors.  Every lane of the wave must
// be active.
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = pair_sum16(pair_sum32(v));
  v += dpp_f<0xB1>(v);     // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);    // row_half_mirror
  v += dpp_f<0x140>(v);    // row_mirror
  return v;
}

// The same exchanges for a float64 value, moved as its two 32-bit halves.
__device__ __forceinline__ double pair_sum32_f64(double v) {
  const uint32_t lo = (uint32_t)__double2loint(v), hi = (uint32_t)__double2hiint(v);
  const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
}

__device__ __forceinline__ double pair_sum16_f64(double v) {
  const uint32_t lo = (uint32_t)__double2loint(v), hi = (uint32_t)__double2hiint(v);
  const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// sum over the wave, the same value left in every lane (every lane active)
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = pair_sum16_f64(pair_sum32_f64(v));
  v += dpp_d<0xB1>(v);
  v += dpp_d<0x4E>(v);
  v += dpp_d<0x141>(v);
  v += dpp_d<0x140>(v);
  return v;
}

// ---------------------------------------------------------------------------
// Activation traffic.  COH = false: plain global accesses (one GEMV per
// launch; the kernel boundary publishes its results).  COH = true: the GEMV
// runs inside a persistent launch and reads what other workgroups of the same
// launch wrote; the per-XCD L2 caches are not coherent with each other, so
// these accesses are system-coherent (sc0 sc1) buffer accesses that bypass
// them.  Weights, gammas and embedding tables are never written and are read
// normally.  Offsets are bytes from the base pointer.
// ---------------------------------------------------------------------------
// Coherent accesses are relaxed atomics at system scope, which the compiler
// emits as plain global loads and stores with the sc0 sc1 bits (no fences);
// 16-byte accesses are two 8-byte halves.
#define M3_COH_LOAD(ptr) __hip_atomic_load((ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
#define M3_COH_STORE(ptr, v) __hip_atomic_store((ptr), (v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)

template <bool COH>
__device__ __forceinline__ uint4 ld16(const void* base, size_t off) {
  const uint8_t* a = static_cast<const uint8_t*>(base) + off;
  if constexpr (COH) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(a);
    const uint64_t lo = M3_COH_LOAD(q), hi = M3_COH_LOAD(q + 1);
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
  } else {
    return *reinterpret_cast<const uint4*>(a);
  }
}

template <bool COH>
__device__ __forceinline__ void st16(void* base, size_t off, const uint4& v) {
  uint8_t* a = static_cast<uint8_t*>(base) + off;
  if constexpr (COH) {
    uint64_t* q = reinterpret_cast<uint64_t*>(a);
    M3_COH_STORE(q, (uint64_t)v.x | ((uint64_t)v.y << 32));
    M3_COH_STORE(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32));
  } else {
    *reinterpret_cast<uint4*>(a) = v;
  }
}

template <bool COH>
__device__ __forceinline__ uint32_t ld4(const void* base, size_t off) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(base) + off);
  if constexpr (COH) return M3_COH_LOAD(a);
  else return *a;
}

template <bool COH>
__device__ __forceinline__ void st4(void* base, size_t off, uint32_t v) {
  uint32_t* a = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + off);
  if constexpr (COH) M3_COH_STORE(a, v);
  else *a = v;
}

template <bool COH>
__device__ __forceinline__ uint32_t ld2(const void* base, size_t off) {
  const uint16_t* a = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(base) + off);
  if constexpr (COH) return M3_COH_LOAD(a);
  else return *a;
}

template <bool COH>
__device__ __forceinline__ void st2(void* base, size_t off, uint32_t v) {
  uint16_t* a = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(base) + off);
  if constexpr (COH) M3_COH_STORE(a, (uint16_t)v);
  else *a = (uint16_t)v;
}

template <bool COH>
__device__ __forceinline__ Best ld_best(const Best* base, size_t i) {
  if constexpr (COH) {
    const uint64_t v = M3_COH_LOAD(reinterpret_cast<const uint64_t*>(base + i));
    return Best{__uint_as_float((uint32_t)v), (int)(uint32_t)(v >> 32)};
  } else {
    return base[i];
  }
}

template <bool COH>
__device__ __forceinline__ void st_best(Best* base, size_t i, const Best& v) {
  if constexpr (COH)
    M3_COH_STORE(reinterpret_cast<uint64_t*>(base + i),
                 (uint64_t)__float_as_uint(v.z) | ((uint64_t)(uint32_t)v.j << 32));
  else
    base[i] = v;
}

// ---------------------------------------------------------------------------
// Tagged activation words (persistent launch).  Inside one persistent launch
// a GEMV's bf16 outputs are 32-bit words: bits 0..15 the value, bits 16..31
// the tag of the phase that wrote it (the low 16 bits of launch * 512 + phase
// + 1).  A consumer reads the words it needs and waits until every tag is the
// one its producer writes, so a dependency costs one store and one load
// instead of a store, a completion wait, a flag store, a flag poll and the
// load.  Stores of 32-bit words are single-copy atomic, so a word with the
// new tag always carries the new value.  No tag newer than the awaited one
// can appear: a phase overwrites a buffer only after every workgroup that
// read it has produced the data that phase waits for.
// ---------------------------------------------------------------------------
constexpr uint32_t kPlain = 0xFFFFFFFFu;   // a plain bf16 buffer (no tags)
constexpr long kSpinLimit = 1L << 21;      // tries (each a memory round trip) before giving up

struct Tags {
  uint32_t x, res, u, part;   // expected tags of the inputs (kPlain: plain buffer)
  uint32_t y;                 // tag of this GEMV's outputs (kPlain: plain outputs)
  uint32_t* err;              // raised when a wait gives up (persistent launch)
};

__device__ __forceinline__ uint32_t tag_of(int producer, uint32_t ebase) {
  return producer < 0 ? kPlain : ((ebase + (uint32_t)producer + 1u) & 0xFFFFu);
}

// Retry loops: spin_more(n, err) is false (and raises *err) once the spin
// limit has passed or another workgroup raised *err, so every wait ends.
__device__ __forceinline__ bool spin_more(long& n, uint32_t* err) {
  if ((++n & 255) == 0 && (n > kSpinLimit || (err && ld4<true>(err, 0) != 0u))) {
    if (err) st4<true>(err, 0, 1u);
    return false;
  }
  return true;
}



__device__ __forceinline__ uint4 untag8(const uint4& a, const uint4& b, uint32_t tag, bool& ok) {
  ok = (a.x >> 16) == tag && (a.y >> 16) == tag && (a.z >> 16) == tag && (a.w >> 16) == tag &&
       (b.x >> 16) == tag && (b.y >> 16) == tag && (b.z >> 16) == tag && (b.w >> 16) == tag;
  return make_uint4((a.x & 0xffffu) | (a.y << 16), (a.z & 0xffffu) | (a.w << 16),
                    (b.x & 0xffffu) | (b.y << 16), (b.z & 0xffffu) | (b.w << 16));
}

// one attempt at elements e .. e+7 of an activation row buffer.  FIRST: a
// first attempt at tagged words through the caches (a workgroup of the same
// XCD may have brought the line in; a stale or torn line fails the tag check
// like an early read), later attempts bypass them
template <bool COH, bool FIRST = false>
__device__ __forceinline__ uint4 act_try8(const void* base, size_t e, uint32_t tag, bool& ok) {
  if constexpr (COH) {
    if (tag != kPlain) {
      const uint4 a = ld16<!FIRST>(base, e * 4), b = ld16<!FIRST>(base, e * 4 + 16);
      return untag8(a, b, tag, ok);
    }
  }
  ok = true;
  return ld16<COH>(base, e * 2);
}

template <bool COH>
__device__ __forceinline__ uint4 act_load8(const void* base, size_t e, uint32_t tag, uint32_t* err) {
  bool ok;
  uint4 v = act_try8<COH, true>(base, e, tag, ok);
  if constexpr (COH) {
    long n = 0;
    while (!ok && spin_more(n, err)) v = act_try8<COH>(base, e, tag, ok);
  }
  return v;
}

template <bool COH>
__device__ __forceinline__ void act_store8(void* base, size_t e, const uint4& v, uint32_t tag) {
  if constexpr (COH) {
    if (tag != kPlain) {
      const uint32_t t = tag << 16;
      st16<true>(base, e * 4, make_uint4((v.x & 0xffffu) | t, (v.x >> 16) | t,
                                         (v.y & 0xffffu) | t, (v.y >> 16) | t));
      st16<true>(base, e * 4 + 16, make_uint4((v.z & 0xffffu) | t, (v.z >> 16) | t,
                                              (v.w & 0xffffu) | t, (v.w >> 16) | t));
      return;
    }
  }
  st16<COH>(base, e * 2, v);
}

template <bool COH>
__device__ __forceinline__ uint32_t act_load1(const void* base, size_t e, uint32_t tag, uint32_t* err) {
  if constexpr (COH) {
    if (tag != kPlain) {
      uint32_t w = ld4<true>(base, e * 4);
      long n = 0;
      while ((w >> 16) != tag && spin_more(n, err)) w = ld4<true>(base, e * 4);
      return w & 0xffffu;
    }
  }
  return ld2<COH>(base, e * 2);
}

template <bool COH>
__device__ __forceinline__ void act_store1(void* base, size_t e, uint32_t bf, uint32_t tag) {
  if constexpr (COH) {
    if (tag != kPlain) {
      st4<true>(base, e * 4, (bf & 0xffffu) | (tag << 16));
      return;
    }
  }
  st2<COH>(base, e * 2, bf);
}

// row-block winners: the column (< 65535; 0xffff = none) with the tag above it
__device__ __forceinline__ Best part_tag(const Best& r, uint32_t tag) {
  if (tag == kPlain) return r;
  const uint32_t j = r.j == 0x7fffffff ? 0xffffu : ((uint32_t)r.j & 0xffffu);
  return Best{r.z, (int)(j | (tag << 16))};
}

template <bool COH>
__device__ __forceinline__ Best part_load(const Best* base, size_t i, uint32_t tag, uint32_t* err) {
  Best r = ld_best<COH>(base, i);
  if constexpr (COH) {
    if (tag != kPlain) {
      long n = 0;
      while (((uint32_t)r.j >> 16) != tag && spin_more(n, err)) r = ld_best<true>(base, i);
      const uint32_t j = (uint32_t)r.j & 0xffffu;
      r.j = j == 0xffffu ? 0x7fffffff : (int)j;
    }
  }
  return r;
}

// source column of operand element k (8-aligned chunk) in x
__device__ __forceinline__ int src_col(const Params& p, int k) {
  if (p.stub_group <= 0) return k;
  return p.stub_voff + (k / (128 * p.stub_group)) * 128 + (k & 127);
}

template <bool COH>
__device__ __forceinline__ uint4 load_x8(const Params& p, int b, int k, const Tags& tg) {
  return act_load8<COH>(p.x, (size_t)b * p.ldx + src_col(p, k), tg.x, tg.err);
}

template <bool COH, bool FIRST = false>
__device__ __forceinline__ uint4 try_x8(const Params& p, int b, int k, const Tags& tg, bool& ok) {
  return act_try8<COH, FIRST>(p.x, (size_t)b * p.ldx + src_col(p, k), tg.x, ok);
}

// Gather prologue: the previous draw of every batch row, from the per-block
// winners the head GEMV wrote (rows b = wave, wave + 8, ... per wave).
template <bool COH>
__device__ __forceinline__ void gather_codes(const Params& p, int* code_lds, int wg, const Tags& tg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const GatherPro& g = p.gat;
  for (int b = wave; b < p.lds_rows; b += kWaves) {
    float bz = -INFINITY;
    int bj = 0x7fffffff;
    for (int c = lane; c < g.nparts; c += 64) {
      const Best r = part_load<COH>(g.part, (size_t)b * g.nparts + c, tg.part, tg.err);
      if (above(r.z, r.j, bz, bj)) {
        bz = r.z;
        bj = r.j;
      }
    }
    best_reduce(bz, bj, 64);
    if (lane == 0) {
      const int32_t id = (g.end_id >= 0 && bj == 0) ? g.end_id : g.index_base + bj;
      code_lds[b] = id;
      if (wg == 0) st4<COH>(g.codes, (size_t)(b * 8 + g.code_col) * 4, (uint32_t)id);
    }
  }
  __syncthreads();
}

// Stage the operand rows in LDS (bf16, row stride lds_stride), fusing the
// norm.  Row b's source is x (with the attention-stub remap) or, in gather
// mode, bf16(u[b] + emb[code_b]).  Three flat passes over all rows so the
// global loads of every row are in flight together: copy (8 chunks of 8
// values per thread per step), per-row sum of squares (one wave per row, a
// fixed order), normalise.
constexpr int kStageUnroll = 8;

__device__ __forceinline__ uint4 bf16x8_add(const uint4& a, const uint4& b) {
  const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = f2bf(bf2f(ua[j] & 0xffffu) + bf2f(ub[j] & 0xffffu)) |
           (f2bf(bf2f(ua[j] >> 16) + bf2f(ub[j] >> 16)) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// One or two rows: the copy also accumulates the sum of squares, spread over
// all threads (row by row; a row's loads are all in flight together).  The
// first kPreRounds chunks per thread and row may have been loaded already
// (XPre): vector-memory loads retire in issue order, so operand loads issued
// after the weight stream would wait for it; issuing them first lets the
// staging overlap the weight stream.
constexpr int kPreRounds = 4;

struct XPre {
  uint4 v[2][kPreRounds];
  bool valid;
};

template <bool COH>
__device__ __forceinline__ void prefetch_x(const Params& p, XPre& pre, const Tags& tg) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < kPreRounds; ++r) {
      const int k = (r * kThreads + tid) << 3;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (b < p.lds_rows && k < p.K) v = load_x8<COH>(p, b, k, tg);
      pre.v[b][r] = v;
    }
  }
  pre.valid = true;
}

// The operand chunk of row b at k (8 values): x (attention-stub remap), or in
// gather mode bf16(u[b] + emb row); k >= K is zero.  try: one attempt (ok =
// the tags matched); settle: until it succeeds.
template <bool COH>
struct OperandSource {
  const Params& p;
  const Tags& tg;
  const int* code_lds;

  __device__ __forceinline__ const uint16_t* emb_row(int b) const {
    int c = code_lds[b] - p.gat.code_base;
    if (c < 0 || c >= p.gat.n_codes) c = 0;
    return p.gat.emb + (size_t)c * p.K;
  }

  template <bool FIRST = false>
  __device__ __forceinline__ uint4 attempt(int b, int k, bool& ok) const {
    ok = true;
    if (k >= p.K) return make_uint4(0, 0, 0, 0);
    if (p.has_gather) {
      const uint4 uv = act_try8<COH, FIRST>(p.gat.u, (size_t)b * p.K + k, tg.u, ok);
      return bf16x8_add(uv, *reinterpret_cast<const uint4*>(emb_row(b) + k));
    }
    return try_x8<COH, FIRST>(p, b, k, tg, ok);
  }

  __device__ __forceinline__ uint4 settle(int b, int k) const {
    bool ok;
    uint4 v = attempt(b, k, ok);
    if constexpr (COH) {
      long n = 0;
      while (!ok && spin_more(n, tg.err)) v = attempt(b, k, ok);
    }
    return v;
  }
};

// The norm's per-row values in the LDS scratch ss_buf (floats): r at
// [0, M3_MAX_B), then (from float offset 2 M3_MAX_B) the few-row path's
// per-wave partial sums of squares (float64).
struct NormLds {
  float* r;
  double* part;
  __device__ explicit NormLds(float* ss_buf)
      : r(ss_buf), part(reinterpret_cast<double*>(ss_buf + 2 * M3_MAX_B)) {}
};

template <bool COH>
__device__ __forceinline__ void stage_rows_few(const Params& p, uint16_t* act, float* ss_buf,
                                               const int* code_lds, int wg, const XPre& pre,
                                               const Tags& tg) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int stride = p.lds_stride;
  const int nchunk = (stride - 8) >> 3;
  const OperandSource<COH> src{p, tg, code_lds};
  NormLds nl(ss_buf);
  auto put = [&](int b, int k, const uint4& v, double& ss) {
    *reinterpret_cast<uint4*>(act + (size_t)b * stride + k) = v;
    if (p.has_gather && wg == 0 && k < p.K) act_store8<COH>(p.gat.out, (size_t)b * p.K + k, v, tg.y);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = sumsq_pair(wv[j], ss);
  };
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (b >= p.lds_rows) break;
    double ss = 0.0;
    if constexpr (!COH) {
      if (pre.valid) {
#pragma unroll
        for (int r = 0; r < kPreRounds; ++r) {
          const int i = r * kThreads + tid;
          if (i < nchunk) put(b, i << 3, pre.v[b][r], ss);
        }
        for (int i = kPreRounds * kThreads + tid; i < nchunk; i += kThreads)
          put(b, i << 3, src.settle(b, i << 3), ss);
      } else {
        for (int i = tid; i < nchunk; i += kThreads) put(b, i << 3, src.settle(b, i << 3), ss);
      }
    } else {
      // request every chunk first, then wait for the ones not yet written
      uint4 v[kPreRounds];
      bool ok[kPreRounds];
#pragma unroll
      for (int r = 0; r < kPreRounds; ++r) {
        const int i = r * kThreads + tid;
        ok[r] = true;
        v[r] = make_uint4(0, 0, 0, 0);
        if (i < nchunk) v[r] = src.template attempt<true>(b, i << 3, ok[r]);
      }
#pragma unroll
      for (int r = 0; r < kPreRounds; ++r) {
        const int k = (r * kThreads + tid) << 3;
        long n = 0;
        while (!ok[r] && spin_more(n, tg.err)) v[r] = src.attempt(b, k, ok[r]);
      }
#pragma unroll
      for (int r = 0; r < kPreRounds; ++r) {
        const int i = r * kThreads + tid;
        if (i < nchunk) put(b, i << 3, v[r], ss);
      }
      for (int i = kPreRounds * kThreads + tid; i < nchunk; i += kThreads)
        put(b, i << 3, src.settle(b, i << 3), ss);
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) nl.part[b * kWaves + wave] = ss;
  }
  __syncthreads();
  if (p.gamma && tid < p.lds_rows) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += nl.part[tid * kWaves + w];
    nl.r[tid] = norm_r(tot, p.K, p.eps);
  }
}

// One launch per GEMV, more than two rows: the first kPreGroups groups of the
// copy pass (kStageUnroll chunks per thread each), requested ahead of the
// weight stream (vector loads retire in issue order: a group requested after
// the first weight batch would wait for it).  Two groups cover 16 rows of
// K = 4096.
constexpr int kPreGroups = 2;
// One launch per GEMV, more than two rows, a fused norm with K <= 4096: gamma
// is requested with the first groups too (two float4 per thread) and kept in
// LDS after the operand rows, so the normalising pass reads no global memory
// and the second weight batch can be requested before the sum of squares.
constexpr int kGammaLdsMaxK = 4 * 2 * kThreads;
struct XGroup {
  uint4 v[kPreGroups][kStageUnroll];
  bool valid;
};
struct GPre {
  float4 g[2];
  bool valid;
};

// LDS bytes of the staged gamma in a one-launch GEMV (0: not staged); the
// host sizes the launch's LDS with it, the kernel decides with it.  Not for
// int8-g128 (its first groups are not prefetched, see gemv_run, and its
// 16-row depth kernels keep two workgroups per CU only without it) nor with
// the gather prologue.
__host__ __device__ inline size_t gamma_lds_bytes(int fmt, bool has_gamma, bool has_gather, int lds_rows,
                                                  int lds_stride, int K, int NB) {
  if (fmt == M3_I8G128 || !has_gamma || has_gather || lds_rows <= 2 || K > kGammaLdsMaxK) return 0;
  const size_t fixed = (size_t)kWaves * NB * 16 * 4 + (size_t)M3_MAX_B * kWaves * 4 + (size_t)M3_MAX_B * 4;
  const size_t need = fixed + (size_t)lds_rows * lds_stride * 2 + (size_t)K * 4;
  return need <= 160 * 1024 ? (size_t)K * 4 : 0;
}

template <bool COH>
__device__ __forceinline__ void prefetch_group(const Params& p, XGroup& g, const Tags& tg, GPre* gp) {
  const int tid = threadIdx.x;
  if (gp) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = u * kThreads + tid;
      gp->g[u] = i * 4 < p.K ? *reinterpret_cast<const float4*>(p.gamma + i * 4) : make_float4(0, 0, 0, 0);
    }
    gp->valid = true;
  }
  const int cpr = (p.lds_stride - 8) >> 3;
  const int total = p.lds_rows * cpr;
#pragma unroll
  for (int q = 0; q < kPreGroups; ++q) {
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int it = tid + (q * kStageUnroll + u) * kThreads;
      const int b = it / cpr, k = (it - b * cpr) * 8;
      const bool in = it < total && k < p.K;
      g.v[q][u] = make_uint4(0, 0, 0, 0);
      if (in) g.v[q][u] = load_x8<COH>(p, b, k, tg);
    }
  }
  g.valid = true;
}

// gl: the LDS gamma of a one-launch GEMV whose gamma was prefetched into
// gp, else nullptr; after_copy() runs once the copy pass is in LDS (there:
// the request of the second weight batch, nothing left to read from global
// memory but the weights)
template <bool COH, class AfterCopy>
__device__ __forceinline__ void stage_activations(const Params& p, uint16_t* act, float* ss_buf,
                                                  int* code_lds, int wg, const XPre& pre,
                                                  const XGroup& grp,
                                                  const Tags& tg, float* gl, const GPre* gp,
                                                  AfterCopy&& after_copy) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int stride = p.lds_stride;
  const int cpr = (stride - 8) >> 3;            // chunks per row: K, padding, zero tile
  const int total = p.lds_rows * cpr;
  if (p.has_gather) gather_codes<COH>(p, code_lds, wg, tg);
  if (p.lds_rows <= 2) {
    stage_rows_few<COH>(p, act, ss_buf, code_lds, wg, pre, tg);
    if (!p.gamma) return;
  } else {
  // pass 1: copy (all requests of a group first; wait for late ones after)
  const OperandSource<COH> src{p, tg, code_lds};
  for (int base = tid; base < total; base += kThreads * kStageUnroll) {
    uint4 v[kStageUnroll];
    bool ok[kStageUnroll];
    const int group = (base - tid) / (kThreads * kStageUnroll);
    if (!COH && grp.valid && group < kPreGroups) {
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        v[u] = group == 0 ? grp.v[0][u] : grp.v[1][u];
        ok[u] = true;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        const int it = base + u * kThreads;
        const int b = it / cpr, k = (it - b * cpr) * 8;
        const bool in = it < total && k < p.K;
        const uint4 x = src.template attempt<true>(in ? b : 0, in ? k : 0, ok[u]);
        v[u] = in ? x : make_uint4(0, 0, 0, 0);
        ok[u] = ok[u] || !in;
      }
    }
    if constexpr (COH) {
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u) {
        const int it = base + u * kThreads;
        const int b = it / cpr, k = (it - b * cpr) * 8;
        long n = 0;
        while (!ok[u] && spin_more(n, tg.err)) v[u] = src.attempt(b, k, ok[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kStageUnroll; ++u) {
      const int it = base + u * kThreads;
      if (it < total) {
        const int b = it / cpr, k = (it - b * cpr) * 8;
        *reinterpret_cast<uint4*>(act + (size_t)b * stride + k) = v[u];
        if (p.has_gather && wg == 0 && k < p.K)
          act_store8<COH>(p.gat.out, (size_t)b * p.K + k, v[u], tg.y);
      }
    }
  }
  if constexpr (!COH) {
    if (gl) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = u * kThreads + tid;
        if (i * 4 < p.K) *reinterpret_cast<float4*>(gl + i * 4) = gp->g[u];
      }
    }
  }
  __syncthreads();
  if constexpr (!COH) {
    if (gl) after_copy();
  }
  if (!p.gamma) return;
  // pass 2: r_b from the sum of squares of row b (float64): lane l sums
  // chunks l + 64 m into accumulator m % 4 (four independent chains whose LDS
  // reads are in flight together), then (s0 + s1) + (s2 + s3), then across
  // the wave
  for (int b = wave; b < p.lds_rows; b += kWaves) {
    const int kc = p.K >> 3;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c0 = lane; c0 < kc; c0 += 256) {
      uint4 v[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int c = c0 + 64 * m;
        v[m] = c < kc ? *reinterpret_cast<const uint4*>(act + (size_t)b * stride + c * 8)
                      : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t wv[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m] = sumsq_pair(wv[j], acc[m]);
      }
    }
    double ss = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    ss = wave_sum_f64(ss);
    if (lane == 0) NormLds(ss_buf).r[b] = norm_r(ss, p.K, p.eps);
  }
  }
  __syncthreads();
  // pass 3: a = bf16(fl32(fl32(x r_b) gamma)) (see norm_pair); gamma is
  // loaded once per chunk
  const NormLds nl(ss_buf);
  const int kc = p.K >> 3;
  for (int i = tid; i < kc; i += kThreads) {
    const int k = i * 8;
    float4 g0, g1;
    if constexpr (!COH) {
      const float* gs = gl ? gl : p.gamma;
      g0 = *reinterpret_cast<const float4*>(gs + k);
      g1 = *reinterpret_cast<const float4*>(gs + k + 4);
    } else {      // (the persistent kernel's code as it was)
      g0 = *reinterpret_cast<const float4*>(p.gamma + k);
      g1 = *reinterpret_cast<const float4*>(p.gamma + k + 4);
    }
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    // rows in groups of four: the group's LDS reads are issued together
    for (int b0 = 0; b0 < p.lds_rows; b0 += 4) {
      uint4 v[4];
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = b0 + e < p.lds_rows ? b0 + e : b0;
        v[e] = *reinterpret_cast<const uint4*>(act + (size_t)b * stride + k);
        r[e] = nl.r[b];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t wv[4] = {v[e].x, v[e].y, v[e].z, v[e].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[j] = norm_pair(wv[j], r[e], g[2 * j], g[2 * j + 1]);
        if (b0 + e < p.lds_rows)
          *reinterpret_cast<uint4*>(act + (size_t)(b0 + e) * stride + k) =
              make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  }
  __syncthreads();
}

// 8 operand values of row b from k; k >= K reads zeros.  Branch-free, so the
// waits for the weight stream are not made conservative by control flow.
template <bool LDS, bool COH>
__device__ __forceinline__ uint4 act8(const Params& p, const uint16_t* act, int b, int k,
                                      const Tags& tg) {
  if constexpr (LDS) {
    return *reinterpret_cast<const uint4*>(act + (size_t)b * p.lds_stride + k);
  } else {
    const bool in = k < p.K;
    const uint4 v = load_x8<COH>(p, b, in ? k : 0, tg);
    return in ? v : make_uint4(0, 0, 0, 0);
  }
}

// Epilogue for one output element (or a gate/up pair) after the cross-wave sum.
template <bool COH>
__device__ __forceinline__ void store_out(const Params& p, int b, int n, float v, const Tags& tg) {
  if (p.out_f32) {
    st4<COH>(p.y, ((size_t)b * p.ldy + n) * 4, __float_as_uint(v));
    return;
  }
  uint32_t o = f2bf(v);
  if (p.epi == M3_EPI_RESIDUAL)
    o = f2bf(bf2f(act_load1<COH>(p.res, (size_t)b * p.ldr + n, tg.res, tg.err)) + bf2f(o));
  act_store1<COH>(p.y, (size_t)b * p.ldy + n, o, tg.y);
}

template <int FMT>
__device__ __forceinline__ float row_scale(const uint8_t* blk, const Params& p, int r) {
  if constexpr (FMT == M3_I8ROW || FMT == M3_FP8ROW)
    return reinterpret_cast<const float*>(blk + (size_t)p.T * kTileBytes)[r];
  return 1.0f;
}

// Cross-wave reduction in fixed wave order, scale, epilogue, store.  GLU: 0
// plain, 1 SwiGLU, 2 chosen at run time by p.epi (one code path for both in
// the persistent kernel, where every compiled variant costs registers).
constexpr int kGluRuntime = 2;

template <int FMT, int NB, int GLU, bool COH>
__device__ __forceinline__ void finish_block(const Params& p, const uint8_t* blk, int rb,
                                             const float* red, const Tags& tg) {
  const int tid = threadIdx.x;
  if (GLU == 1 || (GLU == kGluRuntime && p.epi == M3_EPI_SWIGLU)) {
    for (int t = tid; t < p.B * 8; t += kThreads) {
      const int b = t >> 3, pr = t & 7;
      const int n = rb * 16 + 2 * pr;
      if (n + 1 >= p.N) continue;
      float vg = 0.f, vu = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        vg += red[(w * NB + b) * 16 + 2 * pr];
        vu += red[(w * NB + b) * 16 + 2 * pr + 1];
      }
      vg *= row_scale<FMT>(blk, p, 2 * pr);
      vu *= row_scale<FMT>(blk, p, 2 * pr + 1);
      const float g = bf2f(f2bf(vg)), u = bf2f(f2bf(vu));
      const float s = g / (1.0f + expf(-g));
      act_store1<COH>(p.y, (size_t)b * p.ldy + (n >> 1), f2bf(s * u), tg.y);
    }
    return;
  }
  if (p.has_sample) {
    // logits, then each batch row's best (z, column) over this block's rows;
    // the 16 rows of a batch row are 16 consecutive lanes of one wave
    const SampleEpi& sm = p.smp;
    const uint32_t frame = ld4<COH>(sm.frame, 0);
    const float inv_t = inv_temperature(sm.temperature);
    for (int t0 = 0; t0 < p.B * 16; t0 += kThreads) {
      const int t = t0 + tid;
      const int b = t >> 4, r = t & 15;
      const int n = rb * 16 + r;
      float z = -INFINITY;
      int j = 0x7fffffff;
      if (t < p.B * 16 && n < p.N) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += red[(w * NB + b) * 16 + r];
        v *= row_scale<FMT>(blk, p, r);
        st4<COH>(p.y, ((size_t)b * p.ldy + n) * 4, __float_as_uint(v));
        const int32_t id = (sm.end_id >= 0 && n == 0) ? sm.end_id : sm.index_base + n;
        j = n;
        if (sm.valid_lo < sm.valid_hi && (id < sm.valid_lo || id >= sm.valid_hi) && id != sm.end_id)
          z = -INFINITY;
        else
          z = gumbel_z(v, inv_t, gumbel_noise(sm.seed, (uint32_t)b, frame, sm.draw, (uint32_t)id));
      }
      best_reduce(z, j, 16);
      if (t < p.B * 16 && r == 0)
        st_best<COH>(sm.part, (size_t)b * p.nblocks + rb, part_tag(Best{z, j}, tg.y));
    }
    return;
  }
  for (int t = tid; t < p.B * 16; t += kThreads) {
    const int b = t >> 4, r = t & 15;
    const int n = rb * 16 + r;
    if (n >= p.N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * NB + b) * 16 + r];
    v *= row_scale<FMT>(blk, p, r);
    store_out<COH>(p, b, n, v, tg);
  }
}

// ---------------------------------------------------------------------------
// Weight stream.  Tiles are read with non-temporal 16-byte loads: each weight
// byte is used once per call, so it should not displace the activations and
// partial sums from the caches.
// ---------------------------------------------------------------------------
// Buffer resource over the whole packed matrix (< 2 GiB).  A raw buffer load
// whose VGPR offset is past num_records returns zeros without touching memory;
// adding kOob to a lane's offset turns a load into such a no-op.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes; the uniform part of the address goes in the scalar offset.  AUX is
// the cache policy: non-temporal (2) for weights streamed once per frame (body,
// lm_head); the default (0) for int8-g128, the depth decoder's format, whose
// layers (about 212 MB) are read again at each of the 7 codebook steps of a
// frame and fit in the 256 MB Infinity Cache (measured: 40-55 us less per frame).
template <int AUX>
__device__ __forceinline__ uint4 ldw(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Tiles per batch (KU) is a kernel parameter: 8 for long K slices, 4 where a
// wave's K slice is short (fewer padding tiles).  A wave keeps two batches in
// flight.

// ---------------------------------------------------------------------------
// MFMA accumulators: NB/16 tiles of 16 activation rows.  D[i][j] += sum_k
// A[i][k] B[k][j] with A = activations (row i = lane%16 of a tile), B = the
// weight tile (column j = weight row lane%16); lane l supplies k = 8*(l/16)
// .. +7 of each operand and receives D[4*(l/16) + q][l%16], q = 0..3.
// ---------------------------------------------------------------------------
template <int FMT, int NB>
struct Accum {
  static constexpr int NT = NB / 16;
  f32x4_t acc[NT], gacc[NT];

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) acc[bt] = gacc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  template <bool LDS, bool COH>
  __device__ __forceinline__ void tile(const Params& p, const uint16_t* act, const uint4& wv, int k0,
                                       const Tags& tg) {
    f32x4_t* dst = FMT == M3_I8G128 ? gacc : acc;
    const int lane = threadIdx.x & 63, c = lane >> 4, i = lane & 15;
    if constexpr (FMT == M3_BF16) {
      const int kk = k0 + c * 8;
      const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, wv);
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
        const int b = min(bt * 16 + i, p.B - 1);
        const uint4 av = act8<LDS, COH>(p, act, b, kk, tg);
        dst[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), bw,
                                                          dst[bt], 0, 0, 0);
      }
    } else {
      const int kk = k0 + c * 16;
      uint32_t wb[8];
      bytes16_to_bf16<FMT>(wv, wb);
      const bf16x8_t blo = __builtin_bit_cast(bf16x8_t, make_uint4(wb[0], wb[1], wb[2], wb[3]));
      const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, make_uint4(wb[4], wb[5], wb[6], wb[7]));
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
        const int b = min(bt * 16 + i, p.B - 1);
        const uint4 a0 = act8<LDS, COH>(p, act, b, kk, tg);
        const uint4 a1 = act8<LDS, COH>(p, act, b, kk + 8, tg);
        dst[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), blo,
                                                          dst[bt], 0, 0, 0);
        dst[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), bhi,
                                                          dst[bt], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void group_end(float s) {
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[bt][q] = fmaf(s, gacc[bt][q], acc[bt][q]);
      gacc[bt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  __device__ __forceinline__ void to_red(float* red, int wave) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int bt = 0; bt < NT; ++bt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        red[(wave * NB + bt * 16 + 4 * (lane >> 4) + q) * 16 + (lane & 15)] = acc[bt][q];
  }
};

// Every wave walks the same flat sequence of items (row block, batch of KU
// tiles of its K-slice); item j+2's tiles are requested as soon as item j's
// registers are free, so two batches stay in flight across row-block
// boundaries.  Workgroup wg of nwg owns row blocks wg, wg + nwg, ...
//
// Start-up order.  Vector-memory loads retire in issue order, so whatever is
// requested first is available first.  When the operand is ready (one GEMV
// per launch, or in a persistent launch once the producer has finished), the
// few-row operand is requested first, then one batch of weights, and the
// staging overlaps that batch.  In a persistent launch whose producer is
// still running, two batches of weights are requested before waiting, so the
// wait overlaps the weight stream.  The wait object: probe() (every thread;
// one look at the producer's progress) and wait() (every thread; block until
// the producer is done, false to abandon the GEMV when the launch gives up);
// staged() marks the operand staged (the persistent frame's phase clock).
struct NoWait {
  __device__ bool probe() const { return true; }
  __device__ bool wait() const { return true; }
  __device__ void staged() const {}
  __device__ uint32_t ebase() const { return 0u; }
  __device__ int phase() const { return 0; }
  __device__ uint32_t* err() const { return nullptr; }
};

template <int FMT, int NB, bool LDS, int GLU, int KU, bool COH, class Wait>
__device__ __forceinline__ void gemv_run(const Params& p, uint8_t* smem, int wg, int nwg, Wait&& wt) {
  constexpr int kU = KU;
  static_assert(kU % 2 == 0 && kU <= 16, "batches hold whole i8g128 groups");
  float* red = reinterpret_cast<float*>(smem);                       // [kWaves][NB][16]
  float* ss_buf = red + kWaves * NB * 16;                            // [lds_rows][kWaves]
  int* code_lds = reinterpret_cast<int*>(ss_buf + M3_MAX_B * kWaves);  // [M3_MAX_B]
  uint16_t* act = reinterpret_cast<uint16_t*>(code_lds + M3_MAX_B);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int TPU = FMT == M3_I8G128 ? 2 : 1;    // tiles per unit of the K split
  constexpr int TK = FMT == M3_BF16 ? 32 : 64;     // K elements per tile
  const int units = p.T / TPU;
  const int t_lo = (units * wave / kWaves) * TPU;
  const int ntw = (units * (wave + 1) / kWaves) * TPU - t_lo;       // tiles of this wave
  const int nbat = ((units + kWaves - 1) / kWaves * TPU + kU - 1) / kU;   // same for all waves
  // workgroup wg works as ewg: with follow = the block count F of the phase
  // before (nwg < F < 2 nwg), the workgroups that had one block there (wg >=
  // F - nwg) come first
  int ewg = wg;
  if (p.follow > nwg && p.follow < 2 * nwg) {
    ewg = wg + 2 * nwg - p.follow;
    if (ewg >= nwg) ewg -= nwg;
  }
  const int my_blocks = ewg < p.nblocks ? (p.nblocks - ewg + nwg - 1) / nwg : 0;
  const int nitems = my_blocks * nbat;
  // item j's row block: ewg + (j / nbat) nwg, rotated by rot
  auto block_of = [&](int j) {
    int rb = ewg + (j / nbat) * nwg + p.rot;
    if (rb >= p.nblocks) rb -= p.nblocks;
    return rb;
  };
  Tags tg;
  {
    const uint32_t eb = wt.ebase();
    tg.x = tag_of(p.px, eb);
    tg.res = tag_of(p.pres, eb);
    tg.u = tag_of(p.pu, eb);
    tg.part = tag_of(p.ppart, eb);
    tg.y = p.ytag ? tag_of(wt.phase(), eb) : kPlain;
    tg.err = wt.err();
  }

  // Every wave walks nbat * kU tiles per row block.  Tiles past the end of its
  // K-slice, and the prefetch past the last item, are out-of-range buffer
  // loads (zeros, no memory traffic); their operand is the zero tile, so they
  // add exactly nothing.  The loop has no data-dependent branches, so the
  // compiler's waits let both batches stay in flight.
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(p.w, (uint32_t)((size_t)p.nblocks * p.bbytes));
  const uint32_t vlane = (uint32_t)lane * 16u, vlane_oob = vlane + kOob;
  const int G = p.K / 128;                 // groups per row (i8g128)
  auto load = [&](uint4* dst, float* sc, int j) {
    const bool live = j < nitems;
    const int rb = block_of(j), bi = j % nbat;
    const uint32_t base = (uint32_t)((size_t)rb * p.bbytes) + (uint32_t)t_lo * kTileBytes;
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int tt = bi * kU + i;
      const bool real = live && tt < ntw;
      dst[i] = ldw<FMT == M3_I8G128 ? 0 : 2>(wr, real ? vlane : vlane_oob, real ? base + (uint32_t)tt * kTileBytes : 0u);
    }
    if constexpr (FMT == M3_I8G128) {
      // scales of this batch's kU/2 groups for row lane%16 ([row][group]
      // layout); one dword each so a group past the slice reads a zero
      const uint32_t g0 = (uint32_t)(t_lo + bi * kU) >> 1;
      const uint32_t sbase = (uint32_t)((size_t)rb * p.bbytes) + (uint32_t)p.T * kTileBytes + g0 * 4u;
      const uint32_t vrow = (uint32_t)(lane & 15) * (uint32_t)G * 4u;
#pragma unroll
      for (int q = 0; q < kU / 2; ++q) {
        const bool real = live && bi * kU + 2 * q < ntw;
        sc[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            wr, real ? vrow : vrow + kOob, real ? sbase + 4u * q : 0u, 0));
      }
    }
  };

  Accum<FMT, NB> A;
  A.reset();
  auto compute = [&](const uint4* src, const float* scv, int j) {
    const int rb = block_of(j), bi = j % nbat;
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int tt = bi * kU + i;
      const bool real = tt < ntw;
      A.template tile<LDS, COH>(p, act, src[i], real ? (t_lo + tt) * TK : p.Kp, tg);
      if (FMT == M3_I8G128 && (i & 1)) {
        // groups are tile pairs (t_lo and kU are even): scale the finished group
        A.group_end(real ? scv[i >> 1] : 0.f);
      }
    }
    if (bi == nbat - 1) {          // row block complete: cross-wave sum and epilogue
      A.to_red(red, wave);
      __syncthreads();
      finish_block<FMT, NB, GLU, COH>(p, p.w + (size_t)rb * p.bbytes, rb, red, tg);
      __syncthreads();
      A.reset();
    }
  };

  uint4 bufA[kU], bufB[kU];
  float scA[kU / 2], scB[kU / 2];
  XPre pre;
  pre.valid = false;
  XGroup grp;
  grp.valid = false;
  // one GEMV per launch: the gamma staged in LDS after the operand rows
  GPre gpre;
  gpre.valid = false;
  float* gl = nullptr;
  if constexpr (LDS && !COH) {
    if (gamma_lds_bytes(FMT, p.gamma != nullptr, p.has_gather != 0, p.lds_rows, p.lds_stride, p.K, NB) != 0)
      gl = reinterpret_cast<float*>(act + (size_t)p.lds_rows * p.lds_stride);
  }
  const bool ready = wt.probe();
  if (ready) {
    // (persistent launches: only phase 0, whose operand is plain; not worth the registers)
    if constexpr (LDS && !COH) {
      if (!p.has_gather && nitems > 0) {
        // (not for int8-g128: its 16 extra VGPRs would take the 16-row depth
        // kernels past 128, i.e. from two resident workgroups per CU to one;
        // measured +6..8 us per normed depth GEMV at B = 16)
        if (p.lds_rows <= 2)
          prefetch_x<COH>(p, pre, tg);
        else if constexpr (FMT != M3_I8G128)
          prefetch_group<COH>(p, grp, tg, gl ? &gpre : nullptr);
      }
    }
    load(bufA, scA, 0);
  } else {
    load(bufA, scA, 0);
    load(bufB, scB, 1);
    if (!wt.wait()) return;
  }
  if (nitems == 0) return;
  // with the gamma staged, the second batch is requested once the copy pass
  // is in LDS (the sum of squares and the normalising pass then overlap two
  // batches), else after the staging
  if constexpr (!COH) {
    bool second = false;
    if (LDS)
      stage_activations<COH>(p, act, ss_buf, code_lds, wg, pre, grp, tg, gpre.valid ? gl : nullptr,
                             &gpre, [&]() {
                               load(bufB, scB, 1);
                               second = true;
                             });
    wt.staged();
    if (!second) load(bufB, scB, 1);
  } else {
    if (LDS) stage_activations<COH>(p, act, ss_buf, code_lds, wg, pre, grp, tg, nullptr, nullptr, [] {});
    wt.staged();
    if (ready) load(bufB, scB, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the scheduling barriers keep each batch's loads ahead of the next batch's
  // arithmetic (the scheduler would otherwise sink them into it)
  for (int j = 0; j < nitems; j += 2) {
    compute(bufA, scA, j);
    load(bufA, scA, j + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 >= nitems) break;
    compute(bufB, scB, j + 1);
    load(bufB, scB, j + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One GEMV per launch (the C-ABI entry points and the graph-replayed frame).
// GLU selects the SwiGLU epilogue at compile time (its own kernel symbol, so
// the gate/up GEMVs can be told apart in a profile).
template <int FMT, int NB, bool LDS, bool GLU, int KU>
__global__ __launch_bounds__(kThreads) void gemv_kernel(Params p) {
  extern __shared__ __align__(16) uint8_t smem[];
  gemv_run<FMT, NB, LDS, GLU ? 1 : 0, KU, false>(p, smem, blockIdx.x, gridDim.x, NoWait{});
}

// ---------------------------------------------------------------------------
// Host-side helpers shared by the launch paths.
// ---------------------------------------------------------------------------
// Rows per accumulator tile: the MFMA path in tiles of 16 for every row
// count (rows past B repeat row B-1 and are not stored).  Measured against
// the VALU (dot2) tiles the parameters still express: 5% on the B = 2 frame,
// 0.5% at B = 1, and more from B = 3 on.
inline int nb_of(int B) {
  return (B + 15) / 16 * 16;
}

inline size_t fixed_smem(int NB) {
  return (size_t)kWaves * NB * 16 * 4 + (size_t)M3_MAX_B * kWaves * 4 + (size_t)M3_MAX_B * 4;
}

inline size_t smem_bytes_of(int fmt, int K, int B, bool has_gamma) {
  const size_t fixed = fixed_smem(nb_of(B));
  const size_t act = (size_t)B * (k_pad(fmt, K) + tile_k(fmt) + 8) * 2;
  if (has_gamma || fixed + act <= 160 * 1024) return fixed + act;
  return fixed;
}

// Tiles per batch: 4 for int8-g128 (the depth decoder's short K slices pad
// less), 8 otherwise; operands read from global memory always take 8.  One
// rule for both launch paths, so both run the same sequence of additions.
inline int ku_of(int fmt, bool lds) { return (lds && fmt == M3_I8G128) ? 4 : 8; }

// Kernel parameters of one GEMV (shared by the one-launch and persistent
// paths); also reports whether the activations are staged in LDS and the
// batch size.
inline Params make_params(const GemvDesc& d, bool* lds, int* ku) {
  Params p;
  p.w = static_cast<const uint8_t*>(d.w);
  p.N = d.N;
  p.K = d.K;
  p.Kp = k_pad(d.fmt, d.K);
  p.T = n_tiles(d.fmt, d.K);
  p.nblocks = n_blocks(d.N);
  p.bbytes = block_bytes(d.fmt, d.K);
  p.x = d.x;
  p.ldx = d.ldx;
  p.B = d.B;
  p.gamma = d.gamma;
  p.eps = d.eps;
  p.stub_group = d.stub_group;
  p.stub_voff = d.stub_voff;
  p.y = d.y;
  p.ldy = d.ldy;
  p.out_f32 = d.out_f32;
  p.epi = d.epi;
  p.res = d.res;
  p.ldr = d.ldr;
  const size_t fixed = fixed_smem(nb_of(d.B));
  const size_t smem = smem_bytes_of(d.fmt, d.K, d.B, d.gamma != nullptr);
  *lds = smem > fixed;
  p.lds_rows = *lds ? d.B : 0;
  p.lds_stride = p.Kp + tile_k(d.fmt) + 8;
  p.has_sample = d.sample != nullptr;
  p.has_gather = d.gather != nullptr;
  if (d.sample) p.smp = *d.sample;
  if (d.gather) p.gat = *d.gather;
  p.px = d.px;
  p.pres = d.pres;
  p.pu = d.pu;
  p.ppart = d.ppart;
  p.ytag = d.ytag;
  p.rot = d.rot;
  p.follow = d.follow;
  *ku = ku_of(d.fmt, *lds);
  return p;
}

}  // namespace
}  // namespace m3
