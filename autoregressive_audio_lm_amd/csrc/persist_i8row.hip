// persist_i8row.hip -- persistent frame kernels for a i8row body and lm_head (the
// depth decoder in int8-g128), one per row-count class; see persist.hip.
#include "persist_kernel.h"

namespace m3 {

const void* persist_kernel_i8row(int NB) {
  (void)NB;                 // every row count runs on 16-row tiles
  return reinterpret_cast<const void*>(frame_kernel<16, M3_I8ROW>);
}

}  // namespace m3
