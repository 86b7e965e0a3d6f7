// tiled_half.hip -- instantiations of the tiled kernel for f16 and bf16 a (every tile
// configuration, both b layouts).
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_half(int a_type, int variant, bool bt) {
    switch (a_type) {
    case OUTPROD_TYPE_F16: return tiled_fn<OUTPROD_TYPE_F16>(variant, bt);
    case OUTPROD_TYPE_BF16: return tiled_fn<OUTPROD_TYPE_BF16>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
