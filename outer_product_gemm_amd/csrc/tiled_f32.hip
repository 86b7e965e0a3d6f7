// tiled_f32.hip -- instantiations of the tiled kernel for f32 a (every tile
// configuration, both b layouts) and of the grouped MUL_MAT_ID_BACK
// kernel.
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_f32(int a_type, int variant, bool bt, bool id) {
    switch (a_type) {
    case OUTPROD_TYPE_F32: return id ? id_fn<OUTPROD_TYPE_F32>(variant) : tiled_fn<OUTPROD_TYPE_F32>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
