// tiled_k.hip -- instantiations of the tiled kernel for q3_K, q5_K and q6_K a (every tile
// configuration, both b layouts) and of the grouped MUL_MAT_ID_BACK
// kernel.
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_k(int a_type, int variant, bool bt, bool id) {
    switch (a_type) {
    case OUTPROD_TYPE_Q3_K: return id ? id_fn<OUTPROD_TYPE_Q3_K>(variant) : tiled_fn<OUTPROD_TYPE_Q3_K>(variant, bt);
    case OUTPROD_TYPE_Q5_K: return id ? id_fn<OUTPROD_TYPE_Q5_K>(variant) : tiled_fn<OUTPROD_TYPE_Q5_K>(variant, bt);
    case OUTPROD_TYPE_Q6_K: return id ? id_fn<OUTPROD_TYPE_Q6_K>(variant) : tiled_fn<OUTPROD_TYPE_Q6_K>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
