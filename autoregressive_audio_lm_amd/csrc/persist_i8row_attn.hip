// persist_i8row_attn.hip -- persistent frame kernels for an int8-row body and
// lm_head (the depth decoder in int8-g128) that also carry the attention
// phases (frames with decode attention); see persist.hip and persist_attn.h.
#include "persist_kernel.h"

namespace m3 {

const void* persist_kernel_i8row_attn(bool clock) {
  return clock ? reinterpret_cast<const void*>(frame_kernel<16, M3_I8ROW, true, true>)
               : reinterpret_cast<const void*>(frame_kernel<16, M3_I8ROW, false, true>);
}

}  // namespace m3
