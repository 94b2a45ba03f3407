// persist_fp8row.hip -- persistent frame kernels for an fp8-row body and lm_head
// (the depth decoder in int8-g128), one per row-count class; see persist.hip.
#include "persist_kernel.h"

namespace m3 {

const void* persist_kernel_fp8row(int NB) {
  (void)NB;                 // every row count runs on 16-row tiles
  return reinterpret_cast<const void*>(frame_kernel<16, M3_FP8ROW>);
}

}  // namespace m3
