// kernel_zero.hip -- K == 0: the sum over an empty k range is zero, so dst is
// filled with zeros (dst is overwritten, never accumulated into).
#include "kernel_common.h"
#include "outprod.h"

namespace outprod {
namespace {

__global__ __launch_bounds__(256) void zero_kernel(Problem p, int64_t total) {
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i0 = idx % p.M;
        const int64_t rest = idx / p.M;
        const int64_t i1 = rest % p.N;
        const int64_t z = rest / p.N;
        const int64_t i2 = z % p.ne12, i3 = z / p.ne12;
        *(float *)(p.dst + i3 * p.nb3 + i2 * p.nb2 + i1 * p.nb1 + i0 * 4) = 0.f;
    }
}

}  // namespace

void plan_zero(const Problem &p, Launch *l) {
    const int64_t total = p.M * p.N * p.ne12 * p.ne13;
    int64_t grid = (total + 255) / 256;
    if (grid > 4096) grid = 4096;
    l->kernel = OUTPROD_KERNEL_ZERO;
    l->variant = 0;
    l->tile_m = l->tile_n = l->tile_k = 0;
    l->block = 256;
    l->lds_bytes = 0;
    l->grid = grid;
}

hipError_t launch_zero(const Problem &p, const Launch &l, hipStream_t s) {
    Problem pp = p;
    int64_t total = p.M * p.N * p.ne12 * p.ne13;
    void *args[] = {&pp, &total};
    return hipLaunchKernel((const void *)&zero_kernel, dim3((unsigned)l.grid), dim3(l.block), args,
                           0, s);
}

}  // namespace outprod
