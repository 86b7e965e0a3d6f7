// tiled_q8.hip -- instantiations of the tiled kernel for q8_0, q4_0 and q4_1 a (every tile
// configuration, both b layouts).
#include "tiled_impl.h"

namespace outprod {
namespace tiled {

const void *tiled_kernel_q8(int a_type, int variant, bool bt) {
    switch (a_type) {
    case OUTPROD_TYPE_Q8_0: return tiled_fn<OUTPROD_TYPE_Q8_0>(variant, bt);
    case OUTPROD_TYPE_Q4_0: return tiled_fn<OUTPROD_TYPE_Q4_0>(variant, bt);
    case OUTPROD_TYPE_Q4_1: return tiled_fn<OUTPROD_TYPE_Q4_1>(variant, bt);
    default: return nullptr;
    }
}

}  // namespace tiled
}  // namespace outprod
