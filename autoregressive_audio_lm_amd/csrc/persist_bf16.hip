// persist_bf16.hip -- persistent frame kernels for a bf16 body and lm_head (the
// depth decoder in int8-g128), one per row-count class; see persist.hip.
#include "persist_kernel.h"

namespace m3 {

const void* persist_kernel_bf16(int NB) {
  (void)NB;                 // every row count runs on 16-row tiles
  return reinterpret_cast<const void*>(frame_kernel<16, M3_BF16>);
}

}  // namespace m3
