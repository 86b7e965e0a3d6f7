// tiled_q45.hip -- instantiations of the tiled kernel for q5_0 and q5_1 a (every tile
// configuration, both b layouts) and of the grouped MUL_MAT_ID_BACK
// kernel.
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_q45(int a_type, int variant, bool bt, bool id) {
    switch (a_type) {
    case OUTPROD_TYPE_Q5_0: return id ? id_fn<OUTPROD_TYPE_Q5_0>(variant) : tiled_fn<OUTPROD_TYPE_Q5_0>(variant, bt);
    case OUTPROD_TYPE_Q5_1: return id ? id_fn<OUTPROD_TYPE_Q5_1>(variant) : tiled_fn<OUTPROD_TYPE_Q5_1>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
