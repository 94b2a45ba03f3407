// persist_bf16.hip -- persistent frame kernels for a bf16 body and lm_head
// (the depth decoder in int8-g128): the production kernel and the one that
// also writes the phase clock; see persist.hip.
#include "persist_kernel.h"

namespace m3 {

const void* persist_kernel_bf16(bool clock, bool attn) {
  if (attn) return persist_kernel_bf16_attn(clock);
  return clock ? reinterpret_cast<const void*>(frame_kernel<16, M3_BF16, true>)
               : reinterpret_cast<const void*>(frame_kernel<16, M3_BF16, false>);
}

}  // namespace m3
