// tiled_half.hip -- instantiations of the tiled kernel for f16 and bf16 a (every tile
// configuration, both b layouts) and of the grouped MUL_MAT_ID_BACK
// kernel.
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_half(int a_type, int variant, bool bt, bool id) {
    switch (a_type) {
    case OUTPROD_TYPE_F16: return id ? id_fn<OUTPROD_TYPE_F16>(variant) : tiled_fn<OUTPROD_TYPE_F16>(variant, bt);
    case OUTPROD_TYPE_BF16: return id ? id_fn<OUTPROD_TYPE_BF16>(variant) : tiled_fn<OUTPROD_TYPE_BF16>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
