// persist_fp8row.hip -- persistent frame kernels for an fp8-row body and lm_head
// (the depth decoder in int8-g128): the production kernel and the one that
// also writes the phase clock; see persist.hip.
#include "persist_kernel.h"

namespace m3 {

const void* persist_kernel_fp8row(bool clock, bool attn) {
  if (attn) return persist_kernel_fp8row_attn(clock);
  return clock ? reinterpret_cast<const void*>(frame_kernel<16, M3_FP8ROW, true>)
               : reinterpret_cast<const void*>(frame_kernel<16, M3_FP8ROW, false>);
}

}  // namespace m3
