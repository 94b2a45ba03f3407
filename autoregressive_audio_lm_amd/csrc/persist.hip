// persist.hip -- one whole decode frame as ONE persistent launch.
//
// The frame is a chain of ~270 dependent GEMVs (DiffSynth-Studio
// MiniMax-Music3 stage 2: 36 body layers, the semantic draw, 7 depth-decoder
// steps); launched one per kernel, each pays a launch gap plus a ramp-up and
// a tail during which HBM idles.  Here one workgroup per CU walks a table of
// phases (one GEMV each, then the frame end).  Phase i+1 depends on all of
// phase i, but its weights do not: every workgroup requests its first two
// batches of phase i+1 weight tiles, THEN waits until all workgroups have
// published phase i, so the dependency latency overlaps the weight stream.
//
// Publication: a workgroup finishes its phase-i stores (system-coherent, see
// gemv_impl.h), waits for them to complete, then writes its flag =
// frame * 512 + i + 1 with a coherent store; a waiter's first wave polls all
// flags with coherent loads.  Flags only grow within a frame and from frame to
// frame, and are compared modulo 2^32.  Every wait is bounded: past the spin
// limit the workgroup raises the error word and leaves, and every other
// workgroup leaves at its next poll, so the launch always terminates; the
// host reads the word from the frame state.
//
// The launch is cooperative, so all workgroups are resident at once (the
// waits require it); the launch fails rather than run otherwise.
#include "persist_kernel.h"

#include <cstring>
#include <vector>

namespace m3 {
namespace {

constexpr int kMaxPhases = (int)kPhaseStride - 1;

// A fresh epoch for every recorded phase table: the launch counter advances
// before the flags are set to "phase -1 of it done" and the error word is
// cleared.  Words a launch that gave up left in the tagged streams carry the
// old epoch's tags, which no launch of the new epoch waits for.  (One
// workgroup: every thread reads the counter before thread 0 writes it.)
__global__ void flags_init_kernel(uint32_t* flags, int n, uint32_t* seq, uint32_t* err) {
  const int i = threadIdx.x;
  const uint32_t epoch = *seq + 1u;
  __syncthreads();
  for (int w = i; w < n; w += blockDim.x) flags[w] = epoch * kPhaseStride;
  if (i == 0) {
    *seq = epoch;
    *err = 0u;
  }
}

}  // namespace

// ---- host side ------------------------------------------------------------------
struct PersistPlan {
  std::vector<Phase> phases;
  FeedbackArgs fb{};
  size_t smem = 0;
  int B = 0;
  int fmt_body = -1;      // the kernel's class-0 format
  bool attn = false;      // has attention or guided draw phases (the kernels compiled with them)
};

size_t persist_phase_bytes() { return sizeof(Phase); }
int persist_max_phases() { return kMaxPhases; }

PersistPlan* persist_plan_new(int B) {
  PersistPlan* pl = new PersistPlan;
  pl->B = B;
  return pl;
}

void persist_plan_free(PersistPlan* pl) { delete pl; }

int persist_plan_size(const PersistPlan* pl) { return (int)pl->phases.size(); }

hipError_t persist_add_gemv(PersistPlan* pl, const GemvDesc& d) {
  if ((int)pl->phases.size() >= kMaxPhases || d.B != pl->B) return hipErrorInvalidValue;
  if (d.rot < 0 || d.rot >= n_blocks(d.N) || d.follow < 0) return hipErrorInvalidValue;
  Phase ph{};
  bool lds;
  int ku;
  ph.p = make_params(d, &lds, &ku);
  if (d.gather && !lds) return hipErrorInvalidValue;
  // class 0: the body / lm_head format (bf16 or int8-row, one per frame); class 1: int8-g128
  int cls;
  if (d.fmt == M3_I8G128) {
    cls = 1;
  } else {
    if (pl->fmt_body < 0) pl->fmt_body = d.fmt;
    if (d.fmt != pl->fmt_body) return hipErrorInvalidValue;
    cls = 0;
  }
  // every operand is staged in LDS (the tagged waits happen while staging)
  if (!lds) return hipErrorInvalidValue;
  ph.variant = cls;
  ph.signal = 0;
  const size_t smem = smem_bytes_of(d.fmt, d.K, d.B, d.gamma != nullptr);
  if (smem > pl->smem) pl->smem = smem;
  pl->phases.push_back(ph);
  return hipSuccess;
}

hipError_t persist_add_attention(PersistPlan* pl, const AttnArgs& a) {
  if ((int)pl->phases.size() >= kMaxPhases || a.B != pl->B || a.n_kv < 1) return hipErrorInvalidValue;
  const int g = a.n_q / a.n_kv;
  if (a.n_q != g * a.n_kv || (g != 1 && g != 2 && g != 4) || (a.ch != 64 && a.ch != 128))
    return hipErrorInvalidValue;
  if (a.nchunks < 1 || (long)a.nchunks * a.ch < (long)a.max_pos || (a.nchunks > 1 && !a.rec))
    return hipErrorInvalidValue;
  Phase ph{};
  static_assert(sizeof(AttnArgs) <= sizeof(Params), "attention arguments fit a phase");
  AttnArgs args = a;
  args.scale2 = kLog2e / sqrtf((float)kHD);       // as the decode attention launches
  memcpy(&ph.p, &args, sizeof args);
  ph.variant = kAttnVariant;
  ph.signal = 0;
  const size_t smem = a.ch == 64 ? (g == 1 ? attn_phase_smem<1, 64>() : g == 2 ? attn_phase_smem<2, 64>()
                                                                            : attn_phase_smem<4, 64>())
                                 : (g == 1 ? attn_phase_smem<1, 128>() : g == 2 ? attn_phase_smem<2, 128>()
                                                                              : attn_phase_smem<4, 128>());
  if (smem > pl->smem) pl->smem = smem;
  pl->attn = true;
  pl->phases.push_back(ph);
  return hipSuccess;
}

hipError_t persist_add_cfg(PersistPlan* pl, const CfgDesc& d) {
  if ((int)pl->phases.size() >= kMaxPhases || pl->phases.empty()) return hipErrorInvalidValue;
  if (d.V < 1 || d.V > 36 * kCfgPersistThreads || d.S < 1 || d.S > kPersistFlags / 2 ||
      d.top_k < 1 || !d.part || d.ids || d.noise)
    return hipErrorInvalidValue;
  Phase ph{};
  static_assert(sizeof(CfgDesc) <= sizeof(Params), "draw arguments fit a phase");
  memcpy(&ph.p, &d, sizeof d);
  ph.variant = kCfgVariant;
  ph.signal = 0;
  // the draw waits (on the flags) for every workgroup to finish the logits
  pl->phases.back().signal = 1;
  const size_t smem = sizeof(CfgShared<kCfgPersistThreads>);
  if (smem > pl->smem) pl->smem = smem;
  pl->attn = true;
  pl->phases.push_back(ph);
  return hipSuccess;
}

hipError_t persist_add_feedback(PersistPlan* pl, const uint16_t* tok_emb_audio,
                                const uint16_t* const* audio_emb, int32_t* codes,
                                const Best* last_part, int last_nparts, int32_t vocab_base,
                                int n_slice, int code_vocab, int n_cb, int B, int H,
                                uint16_t* x_out, int32_t* ring, uint32_t* frame,
                                const FeedbackTags& ft) {
  if ((int)pl->phases.size() >= kMaxPhases || pl->phases.empty()) return hipErrorInvalidValue;
  FeedbackArgs& a = pl->fb;
  a.tok = tok_emb_audio;
  for (int i = 0; i < 8; ++i) a.aemb[i] = (i < n_cb - 1) ? audio_emb[i] : nullptr;
  a.codes = codes;
  a.last_part = last_part;
  a.last_nparts = last_nparts;
  a.vocab_base = vocab_base;
  a.n_slice = n_slice;
  a.code_vocab = code_vocab;
  a.n_cb = n_cb;
  a.B = B;
  a.H = H;
  a.x = x_out;
  a.ring = ring;
  a.frame = frame;
  a.last_part_prod = ft.last_part_prod;
  a.th = ft.th;
  a.th_prod = ft.th_prod;
  a.h_out = ft.h_out;
  a.seq = ft.seq;
  a.end_id = ft.end_id;
  a.stop = ft.stop;
  // the frame end waits (on the flags) for every workgroup to finish the step before it
  pl->phases.back().signal = 1;
  Phase ph{};
  ph.variant = kFeedbackVariant;
  ph.signal = 0;
  pl->phases.push_back(ph);
  return hipSuccess;
}

// Persistent launch parameters once the phase table is in device memory.
struct PersistLaunch {
  const void* kernel;          // the production frame kernel
  const void* kernel_clock;    // the same with the phase clock (used while clk is set)
  const Phase* phases;
  int nph;
  uint32_t* flags;
  uint32_t* err;
  const uint32_t* seq;
  FeedbackArgs fb;
  size_t smem;
  int nwg;
  uint64_t* clk = nullptr;   // phase clock buffer, 3 * nph * nwg words (nullptr: off)
};

// Copy the table to `table` (device, persist_phase_bytes() * size), set the
// flags to "phase -1 of the current frame done", clear the error word.
hipError_t persist_upload(const PersistPlan* pl, void* table, uint32_t* flags, uint32_t* err,
                          uint32_t* seq, hipStream_t s, PersistLaunch* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int ncu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int nwg = ncu < kPersistFlags ? ncu : kPersistFlags;
  nwg &= ~3;
  if (nwg < 4) return hipErrorInvalidValue;
  const void* kern[2];
  for (int c = 0; c < 2; ++c) {
    kern[c] = pl->fmt_body == M3_I8ROW    ? persist_kernel_i8row(c != 0, pl->attn)
              : pl->fmt_body == M3_FP8ROW ? persist_kernel_fp8row(c != 0, pl->attn)
                                          : persist_kernel_bf16(c != 0, pl->attn);
    e = hipFuncSetAttribute(kern[c], hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl->smem);
    if (e != hipSuccess) return e;
  }
  e = hipMemcpyAsync(table, pl->phases.data(), pl->phases.size() * sizeof(Phase),
                     hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(flags_init_kernel, dim3(1), dim3(kPersistFlags), 0, s, flags, kPersistFlags,
                     seq, err);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);      // the host table may go away after this
  if (e != hipSuccess) return e;
  out->kernel = kern[0];
  out->kernel_clock = kern[1];
  out->phases = static_cast<const Phase*>(table);
  out->nph = (int)pl->phases.size();
  out->flags = flags;
  out->err = err;
  out->seq = seq;
  out->fb = pl->fb;
  out->smem = pl->smem;
  out->nwg = nwg;
  return hipSuccess;
}

hipError_t persist_launch(const PersistLaunch& L, hipStream_t s) {
  const Phase* ph = L.phases;
  int nph = L.nph;
  uint32_t* flags = L.flags;
  uint32_t* err = L.err;
  const uint32_t* seq = L.seq;
  FeedbackArgs fb = L.fb;
  uint64_t* clk = L.clk;
  void* args[] = {&ph, &nph, &flags, &err, &seq, &fb, &clk};
  return hipLaunchCooperativeKernel(clk ? L.kernel_clock : L.kernel, dim3(L.nwg), dim3(kThreads),
                                    args, (unsigned)L.smem, s);
}

size_t persist_clock_words(const PersistLaunch& L) { return (size_t)3 * L.nph * L.nwg; }
void persist_set_clock(PersistLaunch& L, uint64_t* clk) { L.clk = clk; }
int persist_launch_dims(const PersistLaunch& L, int* nwg) {
  *nwg = L.nwg;
  return L.nph;
}

PersistLaunch* persist_launch_new() { return new PersistLaunch; }
void persist_launch_free(PersistLaunch* L) { delete L; }

}  // namespace m3
