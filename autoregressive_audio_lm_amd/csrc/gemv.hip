// gemv.hip -- one RMSNorm-fused GEMV per launch (the C-ABI GEMV entry points
// and the graph-replayed frame).  The device code lives in gemv_impl.h.
#include "gemv_impl.h"

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

}  // namespace

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
  return hipSuccess;
}

hipError_t launch_gemv(const GemvDesc& d, hipStream_t s) {
  bool lds;
  int ku;      // fixed by the format (see ku_of); the instantiation below follows the same rule
  const Params p = make_params(d, &lds, &ku);
  if (d.gather && !lds) return hipErrorInvalidValue;   // the gather stages through LDS
  const size_t smem = smem_bytes_of(d.fmt, d.K, d.B, d.gamma != nullptr);
  // resident workgroups per CU from LDS (8 waves each, at most 2 per CU)
  int per_cu = (int)((160 * 1024) / (smem + 1024));
  per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
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
