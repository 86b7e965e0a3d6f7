// tiled_q8.hip -- instantiations of the tiled kernel for q8_0, q4_0 and q4_1 a (every tile
// configuration, both b layouts) and of the grouped MUL_MAT_ID_BACK
// kernel.
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_q8(int a_type, int variant, bool bt, bool id) {
    switch (a_type) {
    case OUTPROD_TYPE_Q8_0: return id ? id_fn<OUTPROD_TYPE_Q8_0>(variant) : tiled_fn<OUTPROD_TYPE_Q8_0>(variant, bt);
    case OUTPROD_TYPE_Q4_0: return id ? id_fn<OUTPROD_TYPE_Q4_0>(variant) : tiled_fn<OUTPROD_TYPE_Q4_0>(variant, bt);
    case OUTPROD_TYPE_Q4_1: return id ? id_fn<OUTPROD_TYPE_Q4_1>(variant) : tiled_fn<OUTPROD_TYPE_Q4_1>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
