// prefill.hip -- prompt prefill: RMSNorm over many rows, and the dense GEMM
// Y[M, N] = A[M, K] . W^T on the matrix cores.
//
// A prompt of about 300 tokens for each of the two CFG rows is 600 rows
// through every body matrix at once ("MiniMax Music 3, local": a prompt of
// 300 tokens per CFG row; TensorFold PR #987: 300 tokens a CFG row), a real
// dense contraction: at 600 rows each bf16 weight meets 600 multiply-adds
// (600 flops per byte), above the matrix cores' ridge of about 310 flops per
// byte, so the bound is the MFMA rate, not HBM.
//
// GEMM, two kernels.  Where there are enough tiles of 128 rows (the body's
// QKV and gate/up at 600 rows), the 32 x 32 x 16 MFMA kernel described at
// prefill_mfma32_kernel; elsewhere the following.  A workgroup of 4 waves
// computes a 64 x 128, 96 x 128 or 64 x 256 tile of Y as
// accumulators of v_mfma_f32_16x16x32_bf16; each wave owns a strip of
// columns over all the tile's rows.  The weights stay in the packed tile layout of
// m3_pack: one 16-byte load per lane of a 1 KB tile is exactly the MFMA B
// operand (column = row l % 16 of the block, k = 8 (l / 16) .. +7), so weight
// fragments go from memory straight to registers, each loaded by one wave.
// The A tile (64 rows x 64 K) is staged in LDS (XOR-swizzled, free of bank
// conflicts), shared by the 4 waves and double-buffered; loads run two K
// steps ahead of the MFMAs.
// Tile order: workgroups are handed to the 8 XCDs in turn, so the mapping
// puts the M tiles of one N tile on one XCD in neighbouring slots, where
// they share that XCD's L2 for the weight tiles.
//
// RMSNorm rows: one workgroup per row, a = bf16((x * r) * gamma) with r =
// 1 / sqrt(mean x^2 + eps) in fp32, the same arithmetic as the GEMV prologue.
#include "gemv_impl.h"

namespace m3 {
namespace {

constexpr int kPThreads = 256;                  // 4 waves

// A tile in LDS: rows of 32 KT bf16 (the K step) as 16-byte chunks, chunk ch
// of row r stored at position ch ^ (r % chunks): the 16 lanes of an MFMA
// fragment read (rows r .. r + 15, one chunk) and the 8 lanes that store one
// row hit distinct banks.
template <int KT>
__device__ __forceinline__ int a_off(int r, int ch) {
  constexpr int CH = 4 * KT;
  return r * (8 * CH) + ((ch ^ (r & (CH - 1))) * 8);
}
constexpr int kStages = 3;                      // K steps held in registers (2 in flight)

struct PrefillParams {
  const uint16_t* a;
  int lda;
  const uint8_t* w;
  uint32_t wbytes;
  uint32_t abytes;      // bytes of A from its first row through the end of row M - 1
  uint32_t bbytes;      // bytes per packed row block
  int M, N, K;
  void* y;
  int ldy, out_f32, epi;
  const uint16_t* res;
  int ldr;
  int vec;              // y (and the residual) rows allow 16-byte accesses
  int mtiles, ntiles;
};

// workgroup -> (M tile, N tile), XCD-aware (see above)
__device__ __forceinline__ void tile_of(const PrefillParams& p, int& mt, int& nt) {
  const int nwg = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  int logical = slot;
  for (int x = 0; x < xcd; ++x) logical += (nwg - x + 7) >> 3;   // workgroups on XCD x
  mt = logical % p.mtiles;
  nt = logical / p.mtiles;
}

// Write-out of a wave's staged tile: rows of TR x TC bf16 values (row stride
// SLD) at output rows mw .., columns nw .., as whole 16-byte row chunks, the
// residual read the same way; SwiGLU pairs the interleaved gate/up columns.
template <int EPI, int TR, int TC, int SLD>
__device__ __forceinline__ void store_staged(const PrefillParams& p, const uint16_t* stg, int mw,
                                             int nw, int lane) {
  constexpr int CPR = TC / 8;      // 16-byte chunks per staged row
#pragma unroll
  for (int c = lane; c < TR * CPR; c += 64) {
    const int r = c / CPR, ch = c % CPR;
    const int m = mw + r, n = nw + ch * 8;
    if (m >= p.M || n >= p.N) continue;
    const uint4 v4 = *reinterpret_cast<const uint4*>(&stg[r * SLD + ch * 8]);
    const uint32_t vw[4] = {v4.x, v4.y, v4.z, v4.w};
    const bool whole = p.vec && n + 8 <= p.N;
    if constexpr (EPI == M3_EPI_SWIGLU) {
      // interleaved gate/up rows: staged columns 2t (gate) and 2t + 1 (up)
      // give output column n / 2 + t
      uint16_t* yo = reinterpret_cast<uint16_t*>(p.y) + (size_t)m * p.ldy + (n >> 1);
      uint16_t o[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float g = bf2f(vw[t] & 0xffffu), u = bf2f(vw[t] >> 16);
        o[t] = (uint16_t)f2bf((g / (1.0f + expf(-g))) * u);
      }
      if (whole) {
        *reinterpret_cast<uint2*>(yo) = make_uint2(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16));
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (n + 2 * t < p.N) yo[t] = o[t];
      }
    } else {
      uint16_t* yo = reinterpret_cast<uint16_t*>(p.y) + (size_t)m * p.ldy + n;
      uint32_t ow[4] = {vw[0], vw[1], vw[2], vw[3]};
      if constexpr (EPI == M3_EPI_RESIDUAL) {
        const uint16_t* ro = p.res + (size_t)m * p.ldr + n;
        uint32_t rw[4];
        if (whole) {
          const uint4 r4 = *reinterpret_cast<const uint4*>(ro);
          rw[0] = r4.x; rw[1] = r4.y; rw[2] = r4.z; rw[3] = r4.w;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t lo = n + 2 * t < p.N ? ro[2 * t] : 0u;
            const uint32_t hi = n + 2 * t + 1 < p.N ? ro[2 * t + 1] : 0u;
            rw[t] = lo | (hi << 16);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t lo = f2bf(bf2f(rw[t] & 0xffffu) + bf2f(vw[t] & 0xffffu));
          const uint32_t hi = f2bf(bf2f(rw[t] >> 16) + bf2f(vw[t] >> 16));
          ow[t] = lo | (hi << 16);
        }
      }
      if (whole) {
        *reinterpret_cast<uint4*>(yo) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (n + k < p.N) yo[k] = (uint16_t)(ow[k >> 1] >> (16 * (k & 1)));
      }
    }
  }
}

// A (16 MT WGM) x (16 WNB WGN) tile per workgroup, WGM x WGN = 4 waves.  Wave
// w = (wm, wn) = (w % WGM, w / WGM) holds MT x WNB accumulator tiles of 16 x
// 16: rows 16 MT wm .. +16 MT - 1, columns 16 WNB wn .. +16 WNB - 1.  Each A
// fragment read from LDS feeds WNB MFMAs and each weight fragment MT; with
// WGM = 1 no two waves load the same weight fragment.  Instantiated: <1, 4,
// 2, 2> (64 x 128), <1, 6, 2, 2> (96 x 128) and <1, 4, 4, 2> (64 x 256);
// WGM = 2 and KT = 4 are the measured alternatives the parameters still
// express.
//
// Pipeline over K steps of 32 KT: registers hold the weight fragments and the A
// chunks of three steps; at step ks the loads of step ks + 2 are issued, the
// A chunks of step ks + 1 are written to the LDS buffer that step ks - 1 read,
// and the MFMAs of step ks read LDS buffer ks & 1.  The step count is rounded
// up to a multiple of 3; the extra steps load zeros (offsets past the end of
// the buffers) and add nothing.  A rows past M read zeros the same way.
template <int WGM, int MT, int WNB, int KT, int EPI>
__global__ __launch_bounds__(kPThreads, 2) void prefill_gemm_kernel(PrefillParams p) {
  constexpr int WGN = 4 / WGM;
  constexpr int BM = 16 * MT * WGM, BN = 16 * WNB * WGN;
  constexpr int PK = 32 * KT, CH = PK / 8;       // K step; 16-byte chunks per A row
  constexpr int AC = BM * CH / kPThreads;        // A chunks per thread per K step
  constexpr int KG = MT <= 4 ? 2 : 1;            // K tiles whose A fragments are read at once
  static_assert(AC * kPThreads == BM * CH && KT % KG == 0, "tile shape");
  constexpr int TR = 16 * MT, TC = 16 * WNB, SLD = TC + 8;   // a wave's tile; its staging row stride
  constexpr int LDS_A = 2 * BM * PK, LDS_E = 4 * TR * SLD;
  __shared__ __align__(16) uint16_t lds[LDS_A > LDS_E ? LDS_A : LDS_E];   // A buffers, then the epilogue
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  int mt, nt;
  tile_of(p, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(p.w, p.wbytes);
  const __amdgpu_buffer_rsrc_t ar = weight_rsrc(p.a, p.abytes);
  // this wave's first row block of W; a block past N reads zeros
  const uint32_t wbase = (uint32_t)((n0 >> 4) + WNB * wn) * p.bbytes + (uint32_t)lane * 16u;
  const uint32_t woob = p.wbytes + (uint32_t)lane * 16u;
  uint32_t abase[AC];                            // byte offset of this thread's A chunks at K step 0
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + i * kPThreads, m = m0 + c / CH;
    abase[i] = m < p.M ? (uint32_t)m * (uint32_t)p.lda * 2u + (uint32_t)(c % CH) * 16u : p.abytes;
  }
  const int nk = p.K / PK;
  const int nsteps = (nk + kStages - 1) / kStages * kStages;

  uint4 wreg[kStages][WNB][KT];                  // [stage][row block][K tile]
  uint4 areg[kStages][AC];
  auto load = [&](int st, int ks) {
    const bool in = ks < nk;
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const uint32_t off = wbase + (uint32_t)j * p.bbytes + (uint32_t)(KT * ks + kt) * kTileBytes;
        wreg[st][j][kt] = ldw<0>(wr, in ? off : woob, 0u);
      }
#pragma unroll
    for (int i = 0; i < AC; ++i)
      areg[st][i] = ldw<0>(ar, in ? abase[i] : p.abytes, (uint32_t)ks * (PK * 2));
  };
  auto store_a = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + i * kPThreads;
      *reinterpret_cast<uint4*>(&lds[buf * (BM * PK) + a_off<KT>(c / CH, c % CH)]) = areg[st][i];
    }
  };

  // this lane's A fragment offsets (row 16 MT wm + lane % 16, K chunk 4 kt +
  // lane / 16) in a buffer, for the K tiles of a step
  int aoff[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) aoff[kt] = a_off<KT>(16 * MT * wm + (lane & 15), 4 * kt + (lane >> 4));

  f32x4_t acc[MT][WNB];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(0, 0);
  load(1, 1);
  store_a(0, 0);
  for (int k0 = 0; k0 < nsteps; k0 += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      const int ks = k0 + u;
      load((u + 2) % kStages, ks + 2);
      __builtin_amdgcn_sched_barrier(0);       // keep the loads ahead of this step's MFMAs
      __syncthreads();             // A of step ks is in LDS; the other buffer is free
      const uint16_t* at = &lds[(ks & 1) * (BM * PK)];
      // the A fragments of KG K tiles are read before their MFMAs, so that
      // LDS latency overlaps the matrix work instead of preceding each MFMA
#pragma unroll
      for (int k0t = 0; k0t < KT; k0t += KG) {
        bf16x8_t af[KG][MT];
#pragma unroll
        for (int kt = 0; kt < KG; ++kt)
#pragma unroll
          for (int i = 0; i < MT; ++i)
            af[kt][i] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4*>(at + i * 16 * PK + aoff[k0t + kt]));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < KG; ++kt)
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < WNB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  af[kt][i], __builtin_bit_cast(bf16x8_t, wreg[u][j][k0t + kt]), acc[i][j], 0, 0, 0);
      }
      store_a((u + 1) % kStages, (ks + 1) & 1);
    }
  }

  // epilogue: lane holds D[4 (l / 16) + q][l % 16] of each 16 x 16 tile
  const int mw = m0 + 16 * MT * wm, nw = n0 + 16 * WNB * wn;   // this wave's tile origin
  if constexpr (EPI == M3_EPI_NONE) {
    if (p.out_f32) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = mw + i * 16 + 4 * (lane >> 4) + q, n = nw + j * 16 + (lane & 15);
            if (m < p.M && n < p.N) reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + n] = acc[i][j][q];
          }
      return;
    }
  }
  // bf16 outputs: the wave's tile, rounded to bf16 (every epilogue starts
  // from bf16(acc)), is staged in LDS and leaves as whole 16-byte row chunks,
  // with the residual read the same way
  __syncthreads();                 // every wave is done with the A buffers
  uint16_t* stg = lds + wave * (TR * SLD);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        stg[(i * 16 + 4 * (lane >> 4) + q) * SLD + j * 16 + (lane & 15)] = (uint16_t)f2bf(acc[i][j][q]);
  store_staged<EPI, TR, TC, SLD>(p, stg, mw, nw, lane);
}

// ---------------------------------------------------------------------------
// GEMM on v_mfma_f32_32x32x16_bf16, for the shapes with enough tiles of 128
// rows.  Measured on one MI355X (independent accumulator chains, every CU
// busy): the 32 x 32 x 16 bf16 instruction sustains about 2.46 PFLOP/s, the
// 16 x 16 x 32 one about 1.42, so only the former can approach the bf16 peak.
//
// A workgroup of 4 waves computes a 128 x (64 WNB) tile; wave w holds the
// tile's 128 rows x columns 32 WNB w .. +32 WNB - 1 as 4 x WNB accumulator
// blocks of 32 x 32.  K steps of 32 (one packed weight tile).
//  - A goes to LDS by direct-to-LDS buffer loads (no registers on the way):
//    each step's 128 rows of 64 bytes in a ring of D + 1 slots; a wave load
//    brings 16 rows, every 4 lanes one row's 64 contiguous bytes, the chunk c
//    of row r landing at 16 (c ^ ((r >> 2) & 3)) so that the operand reads
//    (16 lanes: 16 rows, one chunk) hit distinct banks.
//  - The weights go straight to registers, D steps ahead: the B operand of a
//    32 x 32 x 16 MFMA is, per lane, 16 bytes of a packed tile (weight row n
//    = column l % 32 of the block: block n / 16, row n % 16; K 8 (l / 32) ..
//    of the 16-wide half: tile chunk 2 h + l / 32).
//  - Per step: one wait (this wave's loads of the next step's A and of this
//    step's weights; its LDS reads done) and one s_barrier without a memory
//    fence (the fenced barrier would also wait for the loads still in flight
//    for later steps); then the loads of step ks + D, the A operand reads of
//    step ks + 1, and this step's MFMAs, the loads issued between them.
// Rows past M read row M - 1 and weight rows past N read zeros (buffer
// bounds); both are dropped at the write-out.  Padding steps past the last
// load zero weights and add nothing.

// 16 bytes per lane from the buffer at voff + soff into LDS at dst + 16 lane
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff,
                                           uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           soff, 0, 0);
#endif
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N of this wave's vector memory
// loads in flight and none of its LDS accesses
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int WNB, int D, int OCC, int EPI>
__global__ __launch_bounds__(kPThreads, OCC) void prefill_mfma32_kernel(PrefillParams p) {
  constexpr int WMB = 4, BM = 128, BN = 128 * WNB, PK = 32;
  constexpr int S = D + 1;                      // A ring slots and weight register stages
  static_assert(S % 2 == 0, "the A operand registers alternate");
  constexpr int LA = BM / 64;                   // A wave loads per wave per step
  constexpr int SLOT = BM * 64;
  constexpr int LW = 2 * WNB;                   // weight loads per wave per step
  constexpr int TR = 32 * WMB, TC = 32 * WNB, SLD = TC + 8;
  constexpr int LDS_A = S * SLOT, LDS_E = 4 * TR * SLD * 2;
  __shared__ __align__(16) unsigned char lds[LDS_A > LDS_E ? LDS_A : LDS_E];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mt, nt;
  tile_of(p, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(p.w, p.wbytes);
  const __amdgpu_buffer_rsrc_t ar = weight_rsrc(p.a, p.abytes);
  uint32_t wb[WNB];                             // this lane's bytes of block j's B operand, step 0
#pragma unroll
  for (int j = 0; j < WNB; ++j) {
    const int n = n0 + 32 * (WNB * wave + j) + (lane & 31);
    wb[j] = (uint32_t)(n >> 4) * p.bbytes + (uint32_t)((lane & 15) + 16 * (lane >> 5)) * 16u;
  }
  const uint32_t woob = p.wbytes + (uint32_t)lane * 16u;
  uint32_t aoff[LA];                            // this lane's A chunk of each of its wave loads
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    const int r = 16 * (wave * LA + q) + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
    aoff[q] = (uint32_t)min(m0 + r, p.M - 1) * (uint32_t)p.lda * 2u + (uint32_t)c * 16u;
  }
  const int nk = p.K / PK;
  const int nsteps = (nk + S - 1) / S * S;

  uint4 wreg[S][WNB][2];
  auto issue = [&](int st, int ks) {           // the loads of step ks (past nk: zeros, A repeated)
    const bool in = ks < nk;
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wreg[st][j][h] = ldw<0>(wr, in ? wb[j] + (uint32_t)ks * kTileBytes + (uint32_t)h * 512u : woob, 0u);
    const uint32_t soff = (uint32_t)min(ks, nk - 1) * (PK * 2);
#pragma unroll
    for (int q = 0; q < LA; ++q) lds_load16(ar, lds + st * SLOT + (wave * LA + q) * 1024, aoff[q], soff);
  };
  auto read_a = [&](bf16x8_t (&af)[WMB][2], int slot) {
    // block i, half h: row 32 i + l % 32, chunk 2 h + l / 32
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 32 * i + (lane & 31), c = 2 * h + (lane >> 5);
        af[i][h] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(lds + slot * SLOT + r * 64 + 16 * (c ^ ((r >> 2) & 3))));
      }
  };
  f32x16_t acc[WMB][WNB];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8_t afr[2][WMB][2];
#pragma unroll
  for (int u = 0; u < D; ++u) issue(u, u);
  wait_vm_lgkm<(D - 1) * (LA + LW)>();          // step 0's loads are done
  asm volatile("s_barrier" ::: "memory");
  read_a(afr[0], 0);
  for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int ks = k0 + u;
      wait_vm_lgkm<(D - 2) * (LA + LW)>();     // this wave's part of A(ks + 1) and its W(ks)
      asm volatile("s_barrier" ::: "memory");  // every wave's part of A(ks + 1)
      __builtin_amdgcn_sched_barrier(0);
      issue((u + D) % S, ks + D);               // into the slot step ks - 1 read
      read_a(afr[(u + 1) & 1], (u + 1) % S);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < WMB; ++i)
#pragma unroll
          for (int j = 0; j < WNB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                afr[u & 1][i][h], __builtin_bit_cast(bf16x8_t, wreg[u][j][h]), acc[i][j], 0, 0, 0);
      // one load after each of the first MFMAs
#pragma unroll
      for (int q = 0; q < LA + LW; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < 2 * WMB; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vm_lgkm<0>();                            // no LDS write still in flight

  // lane holds D[8 g + 4 (l / 32) + r][l % 32] of each 32 x 32 block in acc[..][4 g + r]
  const int mw = m0, nw = n0 + TC * wave;
  if constexpr (EPI == M3_EPI_NONE) {
    if (p.out_f32) {
#pragma unroll
      for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = mw + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), n = nw + 32 * j + (lane & 31);
            if (m < p.M && n < p.N) reinterpret_cast<float*>(p.y)[(size_t)m * p.ldy + n] = acc[i][j][e];
          }
      return;
    }
  }
  __syncthreads();                 // every wave is done with the A ring
  uint16_t* stg = reinterpret_cast<uint16_t*>(lds) + wave * (TR * SLD);
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        stg[(32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * SLD + 32 * j + (lane & 31)] =
            (uint16_t)f2bf(acc[i][j][e]);
  store_staged<EPI, TR, TC, SLD>(p, stg, mw, nw, lane);
}

template <int WNB, int D, int OCC>
hipError_t launch_mfma32(PrefillParams p, hipStream_t s) {
  constexpr int BM = 128, BN = 128 * WNB;
  p.mtiles = (p.M + BM - 1) / BM;
  p.ntiles = (p.N + BN - 1) / BN;
  const int grid = p.mtiles * p.ntiles;
  if (p.epi == M3_EPI_SWIGLU)
    hipLaunchKernelGGL((prefill_mfma32_kernel<WNB, D, OCC, M3_EPI_SWIGLU>), dim3(grid), dim3(kPThreads), 0, s, p);
  else if (p.epi == M3_EPI_RESIDUAL)
    hipLaunchKernelGGL((prefill_mfma32_kernel<WNB, D, OCC, M3_EPI_RESIDUAL>), dim3(grid), dim3(kPThreads), 0, s, p);
  else
    hipLaunchKernelGGL((prefill_mfma32_kernel<WNB, D, OCC, M3_EPI_NONE>), dim3(grid), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

template <int WGM, int MT, int WNB, int KT>
hipError_t launch_tile(PrefillParams p, hipStream_t s) {
  constexpr int BM = 16 * MT * WGM, BN = 16 * WNB * (4 / WGM);
  p.mtiles = (p.M + BM - 1) / BM;
  p.ntiles = (p.N + BN - 1) / BN;
  const int grid = p.mtiles * p.ntiles;
  if (p.epi == M3_EPI_SWIGLU)
    hipLaunchKernelGGL((prefill_gemm_kernel<WGM, MT, WNB, KT, M3_EPI_SWIGLU>), dim3(grid), dim3(kPThreads), 0, s, p);
  else if (p.epi == M3_EPI_RESIDUAL)
    hipLaunchKernelGGL((prefill_gemm_kernel<WGM, MT, WNB, KT, M3_EPI_RESIDUAL>), dim3(grid), dim3(kPThreads), 0, s, p);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<WGM, MT, WNB, KT, M3_EPI_NONE>), dim3(grid), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

// Tile shape, measured at 600 rows on the body shapes, each GEMM timed inside
// the layer sequence (weights from HBM): 64 x 256 where that still gives
// every CU a tile (gate/up), else 64 x 128, whose 155 registers let three
// workgroups share a CU.  Wider M tiles (128 rows), a 2 x 2 wave arrangement
// (weight fragments loaded twice) and 128-wide K steps all measured slower.
bool wide_tile(int M, int N) {
  return ((M + 63) / 64) * ((N + 255) / 256) >= 256;
}

// 96 x 128 where 64 x 128 tiles would leave some CUs two tiles and 96-row
// tiles give each CU at most one (N = 4096 at 600 rows: 320 tiles -> 224).
// Measured in the layer: down 113 -> 110 us, O unchanged.
bool tall_tile(int M, int N) {
  const int t64 = ((M + 63) / 64) * ((N + 127) / 128), t96 = ((M + 95) / 96) * ((N + 127) / 128);
  return t64 > 256 && t96 <= 256;
}

constexpr int kNThreads = 256;

__global__ __launch_bounds__(kNThreads) void rmsnorm_rows_kernel(const uint16_t* x, int ldx,
                                                                 const float* gamma, float eps,
                                                                 int K, uint16_t* a, int lda) {
  // the decode GEMV prologue's steps (gemv_impl.h, "RMSNorm"): r from a
  // float64 sum of squares, rounded to fp32; two fp32 products per element
  __shared__ double part[kNThreads / 64];
  __shared__ float rs;
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = x + (size_t)row * ldx;
  uint16_t* ar = a + (size_t)row * lda;
  const int kc = K >> 3;
  double ss = 0.0;
  for (int c = tid; c < kc; c += kNThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c * 8);
    ss = sumsq_pair(v.x, ss);
    ss = sumsq_pair(v.y, ss);
    ss = sumsq_pair(v.z, ss);
    ss = sumsq_pair(v.w, ss);
  }
  ss = wave_sum_f64(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) rs = norm_r((part[0] + part[1]) + (part[2] + part[3]), K, eps);
  __syncthreads();
  const float r = rs;
  for (int c = tid; c < kc; c += kNThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c * 8);
    const float4 g0 = *reinterpret_cast<const float4*>(gamma + c * 8);
    const float4 g1 = *reinterpret_cast<const float4*>(gamma + c * 8 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = norm_pair(wv[j], r, g[2 * j], g[2 * j + 1]);
    }
    *reinterpret_cast<uint4*>(ar + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_prefill_gemm(const PrefillDesc& d, hipStream_t s) {
  PrefillParams p{};
  p.a = d.a;
  p.lda = d.lda;
  p.abytes = (uint32_t)(((size_t)(d.M - 1) * d.lda + d.K) * 2);
  p.w = static_cast<const uint8_t*>(d.w);
  p.bbytes = (uint32_t)block_bytes(M3_BF16, d.K);
  p.wbytes = (uint32_t)((size_t)n_blocks(d.N) * p.bbytes);
  p.M = d.M;
  p.N = d.N;
  p.K = d.K;
  p.y = d.y;
  p.ldy = d.ldy;
  p.out_f32 = d.out_f32;
  p.epi = d.epi;
  p.res = d.res;
  p.ldr = d.ldr;
  p.vec = d.ldy % 8 == 0 && (!d.res || (d.ldr % 8 == 0 && reinterpret_cast<uintptr_t>(d.res) % 16 == 0));
  const int mt128 = (d.M + 127) / 128;
  if (d.M >= 256 && mt128 * ((d.N + 255) / 256) >= 384) return launch_mfma32<2, 3, 1>(p, s);
  if (d.M >= 256 && mt128 * ((d.N + 127) / 128) >= 192) return launch_mfma32<1, 5, 2>(p, s);
  if (wide_tile(d.M, d.N)) return launch_tile<1, 4, 4, 2>(p, s);
  if (tall_tile(d.M, d.N)) return launch_tile<1, 6, 2, 2>(p, s);
  return launch_tile<1, 4, 2, 2>(p, s);
}

hipError_t launch_rmsnorm_rows(const uint16_t* x, int M, int K, int ldx, const float* gamma,
                               float eps, uint16_t* a, int lda, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(M), dim3(kNThreads), 0, s, x, ldx, gamma, eps, K, a,
                     lda);
  return hipGetLastError();
}

}  // namespace m3
