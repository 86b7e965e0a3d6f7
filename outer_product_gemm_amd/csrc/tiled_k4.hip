// tiled_k4.hip -- instantiations of the tiled kernel for q4_K and q2_K a (every tile
// configuration, both b layouts) and of the grouped MUL_MAT_ID_BACK
// kernel.
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_k4(int a_type, int variant, bool bt, bool id) {
    switch (a_type) {
    case OUTPROD_TYPE_Q4_K: return id ? id_fn<OUTPROD_TYPE_Q4_K>(variant) : tiled_fn<OUTPROD_TYPE_Q4_K>(variant, bt);
    case OUTPROD_TYPE_Q2_K: return id ? id_fn<OUTPROD_TYPE_Q2_K>(variant) : tiled_fn<OUTPROD_TYPE_Q2_K>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
