// noalloc.hip -- out_prod_noalloc: out_prod for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs out_prod's own plan; a
// plan that splits K writes its partials to `scratch`, a fixed array in the
// library's device image, instead of a workspace of the pool.
#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include "outprod.h"
#include "outprod_internal.h"

// The split partials of out_prod_noalloc.  Each device holds its own copy,
// loaded with the library's code object, until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: host
// code uses the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[outprod::kScratchBytes];

namespace outprod {
namespace {

struct ScratchAddr {
    int device;
    uint8_t *ptr;
};
std::mutex g_scratch_mutex;
std::vector<ScratchAddr> g_scratch;

// The device address of this device's `scratch`, looked up once per device
// (with the device current) on its first call.
int scratch_ptr(uint8_t **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return OUTPROD_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    for (const ScratchAddr &s : g_scratch) {
        if (s.device == dev) {
            *out = s.ptr;
            return OUTPROD_OK;
        }
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return OUTPROD_E_HIP;
    g_scratch.push_back(ScratchAddr{dev, (uint8_t *)ptr});
    *out = (uint8_t *)ptr;
    return OUTPROD_OK;
}

}  // namespace
}  // namespace outprod

extern "C" int out_prod_noalloc(const void *a, int a_type, const float *b, float *dst,
                                const int64_t ne[12], const int64_t nb[12], void *stream) {
    outprod::Checked c;
    int rc = outprod::validate_and_plan(a, a_type, b, dst, ne, nb, OUTPROD_KERNEL_AUTO, &c);
    if (rc != OUTPROD_OK) return rc;
    uint8_t *ws = nullptr;
    if (c.l.splits > 1) {
        if (outprod::split_bytes(c.p, c.l.splits) > outprod::kScratchBytes) return OUTPROD_E_SCRATCH;
        rc = outprod::scratch_ptr(&ws);
        if (rc != OUTPROD_OK) return rc;
    }
    return outprod::enqueue(c, (hipStream_t)stream, ws) == hipSuccess ? OUTPROD_OK : OUTPROD_E_HIP;
}
