// api.cpp -- the C entry points of liboutprod.so: host-side validation of the
// OUT_PROD contract, kernel planning and the single launch.
//
// The contract (pages: "metal: OUT_PROD runs batched, broadcast and narrow
// shapes on the GPU", review "VERIFIED BY READING"): dst is {a.ne0, b.ne0,
// b.ne2, b.ne3}; b.ne2 % a.ne2 == 0 and b.ne3 % a.ne3 == 0; slice i2 of dst
// reads a slice i2/dps2.  The same page's body scopes the width rule to the
// quantized copy only, so an f32 a of any width is accepted and a quantized a
// needs only whole blocks.  Unsupported problems are refused with a status
// code before any HIP call; there is no silent fallback.
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "outprod.h"
#include "outprod_internal.h"

namespace outprod {
namespace {

// Values and bytes per block of each a type (0 bytes: unknown type).
struct TypeInfo {
    int values, bytes;
};
TypeInfo type_info(int t) {
    switch (t) {
    case OUTPROD_TYPE_F32: return {1, 4};
    case OUTPROD_TYPE_F16: return {1, 2};
    case OUTPROD_TYPE_BF16: return {1, 2};
    case OUTPROD_TYPE_Q4_0: return {32, 18};
    case OUTPROD_TYPE_Q4_1: return {32, 20};
    case OUTPROD_TYPE_Q5_0: return {32, 22};
    case OUTPROD_TYPE_Q5_1: return {32, 24};
    case OUTPROD_TYPE_Q8_0: return {32, 34};
    case OUTPROD_TYPE_Q2_K: return {256, 84};
    case OUTPROD_TYPE_Q3_K: return {256, 110};
    case OUTPROD_TYPE_Q4_K: return {256, 144};
    case OUTPROD_TYPE_Q5_K: return {256, 176};
    case OUTPROD_TYPE_Q6_K: return {256, 210};
    default: return {0, 0};
    }
}
int block_values(int t) { return type_info(t).values; }
int block_bytes(int t) { return type_info(t).bytes; }
// a's pointer and strides: 4-byte aligned when the element or block size is a
// multiple of 4 (the kernels read such blocks with 32-bit loads), else 2
int align_of(int t) { return block_bytes(t) % 4 == 0 ? 4 : 2; }

// x*y + z for non-negative int64, false on overflow.
bool mul_add(int64_t x, int64_t y, int64_t z, int64_t *out) {
    __int128 r = (__int128)x * y + z;
    if (r > INT64_MAX) return false;
    *out = (int64_t)r;
    return true;
}

// Bytes spanned by a 4-d view: last byte offset + 1.  dim0_bytes is the byte
// length of one row along dim 0.  False on overflow.
bool extent(int64_t dim0_bytes, const int64_t *ne, const int64_t *nb, int64_t *out) {
    int64_t e = dim0_bytes;
    for (int d = 1; d < 4; ++d)
        if (ne[d] > 1 && !mul_add(ne[d] - 1, nb[d], e, &e)) return false;
    *out = e;
    return true;
}

bool overlaps(const void *p, int64_t np, const void *q, int64_t nq) {
    if (np <= 0 || nq <= 0) return false;
    uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)np;
    uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)nq;
    return a0 < b1 && b0 < a1;
}

// The same OUT_PROD with the roles of a and b exchanged: dst^T = a'·b'^T with
// a' = b, b' = a, so dst element (i0, i1) is element (i1, i0) of the swapped
// problem (dst strides exchanged).  Used for a narrow f32 b (ne10 <= 32) with a
// wide f32 a, e.g. the gradient of a LoRA down-projection out_prod(x, grad_h),
// so the column kernel can stream the wide operand.  The slice broadcast
// stays on the original a, which is now the kernel's b.
Problem swap_operands(const Problem &p) {
    Problem q = p;
    q.a = p.b;
    q.b = p.a;
    q.M = p.N;
    q.N = p.M;
    q.nb01 = p.nb11;
    q.nb02 = p.nb12;
    q.nb03 = p.nb13;
    q.nb10 = 4;
    q.nb11 = p.nb01;
    q.nb12 = p.nb02;
    q.nb13 = p.nb03;
    q.nb0 = p.nb1;
    q.nb1 = p.nb0;
    q.vec_a = p.vec_b;
    q.vec_b = p.vec_a;
    q.b_kt = false;
    q.bcast_b = true;
    return q;
}

}  // namespace

// no_split: plan without a K split unless one is forced (for a call that
// has no workspace).
int validate_and_plan(const void *a, int a_type, const float *b, const float *dst,
                      const int64_t *ne, const int64_t *nb, int kernel, Checked *c,
                      bool no_split) {
    if (!ne || !nb) return OUTPROD_E_NULL;
    if (block_bytes(a_type) == 0) return OUTPROD_E_TYPE;
    for (int i = 0; i < 12; ++i)
        if (ne[i] < 0) return OUTPROD_E_SHAPE;
    const int64_t ne00 = ne[0], K = ne[1], ne02 = ne[2], ne03 = ne[3];
    const int64_t ne10 = ne[4], ne12 = ne[6], ne13 = ne[7];
    if (ne[5] != K) return OUTPROD_E_K;
    if (ne[8] != ne00 || ne[9] != ne10 || ne[10] != ne12 || ne[11] != ne13)
        return OUTPROD_E_DST_SHAPE;

    memset(c, 0, sizeof(*c));
    Problem &p = c->p;
    Launch &l = c->l;
    p.a_type = a_type;
    p.M = ne00;
    p.N = ne10;
    p.K = K;
    p.ne12 = ne12;
    p.ne13 = ne13;

    const bool empty = ne00 == 0 || ne10 == 0 || ne12 == 0 || ne13 == 0;
    if (empty) {
        const int fam = kernel & 0xFF;
        if (fam != OUTPROD_KERNEL_AUTO && fam != OUTPROD_KERNEL_SKINNY && fam != OUTPROD_KERNEL_TILED)
            return OUTPROD_E_KERNEL;
        l.kernel = OUTPROD_KERNEL_NONE;
        return OUTPROD_OK;
    }

    if (ne02 < 1 || ne03 < 1 || ne12 % ne02 != 0 || ne13 % ne03 != 0) return OUTPROD_E_BCAST;
    p.dps2 = ne12 / ne02;
    p.dps3 = ne13 / ne03;

    if (ne00 % block_values(a_type) != 0) return OUTPROD_E_QK;

    // strides and alignment
    // b is either row-major (dim 0 contiguous, nb10 == 4) or K-contiguous
    // (nb11 == 4: a transposed view such as the gradient grad^T that the
    // matmul backward passes for the input gradient); a and dst have dim 0
    // contiguous.
    if (nb[0] != block_bytes(a_type) || nb[8] != 4) return OUTPROD_E_LAYOUT;
    for (int i = 0; i < 12; ++i)
        if (nb[i] < 0) return OUTPROD_E_LAYOUT;
    const bool b_rows = nb[4] == 4;
    if (!b_rows && nb[5] != 4) return OUTPROD_E_LAYOUT;
    const int al = align_of(a_type);
    if (nb[4] % 4 != 0) return OUTPROD_E_LAYOUT;
    for (int i = 1; i < 4; ++i)
        if (nb[i] % al != 0 || nb[4 + i] % 4 != 0 || nb[8 + i] % 4 != 0) return OUTPROD_E_LAYOUT;
    if ((uintptr_t)a % al != 0 || (uintptr_t)b % 4 != 0 || (uintptr_t)dst % 4 != 0)
        return OUTPROD_E_LAYOUT;
    // dst dims must be ordered and disjoint so that every element has one address
    {
        int64_t span = 4 * ne00;  // bytes of one dst row
        for (int d = 1; d < 4; ++d) {
            if (ne[8 + d] > 1) {
                if (nb[8 + d] < span) return OUTPROD_E_LAYOUT;
                if (!mul_add(ne[8 + d] - 1, nb[8 + d], span, &span)) return OUTPROD_E_RANGE;
            }
        }
    }

    if (!dst) return OUTPROD_E_NULL;
    if (K > 0 && (!a || !b)) return OUTPROD_E_NULL;

    // index range: the kernels index workgroups, rows and columns with 32-bit ints
    const int64_t lim = INT32_MAX;
    int64_t slices;
    if (!mul_add(ne12, ne13, 0, &slices) || slices > lim || ne00 > lim || ne10 > lim || K > lim)
        return OUTPROD_E_RANGE;
    const int64_t a_row = ne00 / block_values(a_type) * block_bytes(a_type);
    int64_t ext_a = 0, ext_b = 0, ext_d = 0;
    if (K > 0) {
        const int64_t ane[4] = {ne00, K, ne02, ne03}, anb[4] = {nb[0], nb[1], nb[2], nb[3]};
        // b: last byte = 4 + sum over its four dims of (ne - 1) * nb (either dim
        // 0 or dim 1 may be the contiguous one)
        const int64_t bne[4] = {ne10, K, ne12, ne13}, bnb[4] = {nb[4], nb[5], nb[6], nb[7]};
        if (!extent(a_row, ane, anb, &ext_a) || !mul_add(ne10 - 1, nb[4], 4, &ext_b) ||
            !extent(ext_b, bne, bnb, &ext_b))
            return OUTPROD_E_RANGE;
    }
    {
        const int64_t dne[4] = {ne00, ne10, ne12, ne13}, dnb[4] = {4, nb[9], nb[10], nb[11]};
        if (!extent(4 * ne00, dne, dnb, &ext_d)) return OUTPROD_E_RANGE;
    }
    if (K > 0 && (overlaps(dst, ext_d, a, ext_a) || overlaps(dst, ext_d, b, ext_b)))
        return OUTPROD_E_ALIAS;

    p.a = (const uint8_t *)a;
    p.b = (const uint8_t *)b;
    p.dst = (uint8_t *)dst;
    p.nb01 = nb[1];
    p.nb02 = nb[2];
    p.nb03 = nb[3];
    p.nb10 = nb[4];
    p.nb11 = nb[5];
    p.b_kt = !b_rows;
    p.nb0 = 4;
    p.nb12 = nb[6];
    p.nb13 = nb[7];
    p.nb1 = nb[9];
    p.nb2 = nb[10];
    p.nb3 = nb[11];
    // 16-byte vector loads of a's rows (f32: 4 values, f16/bf16: 8 values)
    p.vec_a = (a_type == OUTPROD_TYPE_F32 || a_type == OUTPROD_TYPE_F16 ||
               a_type == OUTPROD_TYPE_BF16) &&
              (uintptr_t)a % 16 == 0 && nb[1] % 16 == 0 && nb[2] % 16 == 0 && nb[3] % 16 == 0;
    // 16-byte vector loads of b: along its contiguous dim, so the other
    // strides must keep 16-byte alignment
    p.vec_b = (uintptr_t)b % 16 == 0 && (b_rows ? nb[5] : nb[4]) % 16 == 0 && nb[6] % 16 == 0 &&
              nb[7] % 16 == 0;

    if (K == 0) {
        const int fam = kernel & 0xFF;
        if (fam != OUTPROD_KERNEL_AUTO && fam != OUTPROD_KERNEL_SKINNY && fam != OUTPROD_KERNEL_TILED)
            return OUTPROD_E_KERNEL;
        plan_zero(p, &l);
        return l.grid > lim ? OUTPROD_E_RANGE : OUTPROD_OK;
    }

    // kernel = family | (tile configuration + 1) << 8 | splits << 16 |
    // group_m << 24; configuration 0, splits 0 and group_m 0 = automatic
    const int variant = (kernel >> 8) & 0xFF;
    const int splits = (kernel >> 16) & 0xFF;
    const int group_m = (kernel >> 24) & 0x7F;
    kernel &= 0xFF;
    if ((variant != 0 || splits != 0) && kernel != OUTPROD_KERNEL_TILED &&
        kernel != OUTPROD_KERNEL_SKINNY)
        return OUTPROD_E_KERNEL;
    if (group_m != 0 && kernel != OUTPROD_KERNEL_TILED) return OUTPROD_E_KERNEL;
    l.group_m = group_m;
    l.variant = variant;
    l.splits = splits == 0 && no_split ? 1 : splits;
    bool ok;
    switch (kernel) {
    case OUTPROD_KERNEL_AUTO: {
        // narrow f32 a, or an f32 problem with too few output tiles to fill
        // the chip: the column kernel; a narrow row-major b with a wide f32 a:
        // the column kernel on the operand-swapped problem; everything else:
        // the tiled kernel
        Launch t = l;
        const bool tiled_ok = plan_tiled(p, &t);
        const bool f32 = p.a_type == OUTPROD_TYPE_F32;
        if (f32 && p.M <= 32) {
            ok = plan_skinny(p, &l);
        } else if (f32 && p.N <= 32 && !p.b_kt) {
            c->p = swap_operands(p);
            c->swapped = true;
            ok = plan_skinny(c->p, &l);
        } else if (f32 && (!tiled_ok || t.grid / t.splits < 128)) {
            // (output tiles counted without K splits)
            ok = plan_skinny(p, &l);
        } else {
            l = t;
            ok = tiled_ok;
        }
        break;
    }
    case OUTPROD_KERNEL_SKINNY:
        ok = plan_skinny(p, &l);
        break;
    case OUTPROD_KERNEL_TILED:
        ok = plan_tiled(p, &l);
        break;
    default:
        ok = false;
    }
    if (!ok) return OUTPROD_E_KERNEL;
    if (l.grid > lim) return OUTPROD_E_RANGE;
    return OUTPROD_OK;
}

hipError_t enqueue(Checked &c, hipStream_t s, uint8_t *ws) {
    if (c.l.splits > 1) {
        c.p.splits = c.l.splits;
        c.p.ksplit = c.l.ksplit;
        c.p.ws = ws;
    }
    hipError_t e = hipSuccess;
    switch (c.l.kernel) {
    case OUTPROD_KERNEL_NONE:
        return hipSuccess;
    case OUTPROD_KERNEL_ZERO:
        e = launch_zero(c.p, c.l, s);
        break;
    case OUTPROD_KERNEL_SKINNY:
        e = launch_skinny(c.p, c.l, s);
        break;
    case OUTPROD_KERNEL_TILED:
        e = launch_tiled(c.p, c.l, s);
        break;
    default:
        return hipErrorInvalidValue;
    }
    if (e == hipSuccess && c.p.splits > 1) e = launch_split_reduce(c.p, s);
    return e;
}

namespace {

// The library's workspaces (split-K partials, MUL_MAT_ID_BACK routing
// tables): at most kMaxWorkspaces per device, kWorkspaceBytes each, each
// bound to one stream.  A stream's first call that needs one allocates it
// (never under capture), and it stays bound -- a graph captured on the stream
// keeps its address -- until out_prod_release_stream frees it.  So the
// library holds at most kMaxWorkspaces * kWorkspaceBytes per device however
// many streams come and go.
struct Workspace {
    int device;
    hipStream_t stream;
    uint8_t *ptr;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;

// The workspace of `stream` on the current device, allocated on its first
// use.  OUTPROD_E_WORKSPACE: the device already has kMaxWorkspaces, bound to
// other streams; OUTPROD_E_CAPTURE: the stream has none and is capturing (an
// allocation would invalidate the capture).
int stream_workspace(hipStream_t stream, uint8_t **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return OUTPROD_E_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int on_dev = 0;
    for (const Workspace &w : g_ws) {
        if (w.device != dev) continue;
        ++on_dev;
        if (w.stream == stream) {
            *out = w.ptr;
            return OUTPROD_OK;
        }
    }
    if (on_dev >= kMaxWorkspaces) return OUTPROD_E_WORKSPACE;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return OUTPROD_E_HIP;
    if (st != hipStreamCaptureStatusNone) return OUTPROD_E_CAPTURE;
    void *ptr = nullptr;
    if (hipMalloc(&ptr, (size_t)kWorkspaceBytes) != hipSuccess) return OUTPROD_E_HIP;
    g_ws.push_back(Workspace{dev, stream, (uint8_t *)ptr});
    *out = (uint8_t *)ptr;
    return OUTPROD_OK;
}

// Free the workspace of `stream` (for the NULL stream: the current
// device's) once the stream's queued work has finished with it.
int release_stream(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return OUTPROD_E_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    size_t i = 0;
    while (i < g_ws.size() && !(g_ws[i].stream == stream && (stream != nullptr || g_ws[i].device == dev)))
        ++i;
    if (i == g_ws.size()) return OUTPROD_OK;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return OUTPROD_E_HIP;
    if (st != hipStreamCaptureStatusNone) return OUTPROD_E_CAPTURE;
    const Workspace w = g_ws[i];
    if (w.device != dev && hipSetDevice(w.device) != hipSuccess) return OUTPROD_E_HIP;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipFree(w.ptr);
    if (w.device != dev) (void)hipSetDevice(dev);
    if (e != hipSuccess) return OUTPROD_E_HIP;
    g_ws.erase(g_ws.begin() + (std::ptrdiff_t)i);
    return OUTPROD_OK;
}

int run(const void *a, int a_type, const float *b, float *dst, const int64_t *ne,
        const int64_t *nb, void *stream, int kernel) {
    Checked c;
    int rc = validate_and_plan(a, a_type, b, dst, ne, nb, kernel, &c);
    if (rc != OUTPROD_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = nullptr;
    if (c.l.splits > 1) {
        rc = stream_workspace(s, &ws);
        if (rc == OUTPROD_E_CAPTURE || rc == OUTPROD_E_WORKSPACE) {
            // no workspace for this stream: an automatic plan runs unsplit
            // instead (the same sum in another order; a forced split fails)
            if ((kernel >> 16) & 0xFF) return rc;
            rc = validate_and_plan(a, a_type, b, dst, ne, nb, kernel, &c, true);
            if (rc != OUTPROD_OK) return rc;
        } else if (rc != OUTPROD_OK) {
            return rc;
        }
    }
    return enqueue(c, s, ws) == hipSuccess ? OUTPROD_OK : OUTPROD_E_HIP;
}

// ---------------------------------------------------------------- MUL_MAT_ID_BACK

struct IdChecked {
    IdProblem p;
    Launch l;
    bool zero;  // K == 0: dst rows are zeros, no routing
};

// ne/nb[16]: as {ne00, K, n_expert, 1}, g {K, n_used, n_tokens, 1}, ids
// {n_used, n_tokens, 1, 1}, dst {ne00, n_used, n_tokens, 1}.
int validate_id_back(const void *as, int as_type, const float *g, const int32_t *ids,
                     const float *dst, const int64_t *ne, const int64_t *nb, int kernel,
                     IdChecked *c) {
    if (!ne || !nb) return OUTPROD_E_NULL;
    if (block_bytes(as_type) == 0) return OUTPROD_E_TYPE;
    for (int i = 0; i < 16; ++i)
        if (ne[i] < 0) return OUTPROD_E_SHAPE;
    const int64_t ne00 = ne[0], K = ne[1], E = ne[2], n_used = ne[5], n_tok = ne[6];
    if (ne[4] != K) return OUTPROD_E_K;
    if (ne[3] != 1 || ne[7] != 1 || ne[8] != n_used || ne[9] != n_tok || ne[10] != 1 || ne[11] != 1)
        return OUTPROD_E_SHAPE;
    if (ne[12] != ne00 || ne[13] != n_used || ne[14] != n_tok || ne[15] != 1) return OUTPROD_E_DST_SHAPE;

    memset(c, 0, sizeof(*c));
    IdProblem &p = c->p;
    Launch &l = c->l;
    p.a_type = as_type;
    p.M = ne00;
    p.K = K;
    p.n_expert = E;
    p.n_used = n_used;
    p.n_tokens = n_tok;
    const int64_t slots = n_used * n_tok;
    if (ne00 == 0 || slots == 0) {
        const int fam = kernel & 0xFF;
        if (fam != OUTPROD_KERNEL_AUTO && fam != OUTPROD_KERNEL_TILED) return OUTPROD_E_KERNEL;
        l.kernel = OUTPROD_KERNEL_NONE;
        return OUTPROD_OK;
    }
    if (K > 0 && E < 1) return OUTPROD_E_BCAST;  // no expert to route to
    if (ne00 % block_values(as_type) != 0) return OUTPROD_E_QK;

    // layout: dim 0 of each tensor contiguous; 4-byte strides (2 for the
    // experts of 2-byte aligned types); dst rows ordered and disjoint
    if (nb[0] != block_bytes(as_type) || nb[4] != 4 || nb[8] != 4 || nb[12] != 4) return OUTPROD_E_LAYOUT;
    for (int i = 0; i < 16; ++i)
        if (nb[i] < 0) return OUTPROD_E_LAYOUT;
    const int al = align_of(as_type);
    if (nb[1] % al || nb[2] % al || nb[5] % 4 || nb[6] % 4 || nb[9] % 4 || nb[13] % 4 || nb[14] % 4)
        return OUTPROD_E_LAYOUT;
    if ((uintptr_t)as % al || (uintptr_t)g % 4 || (uintptr_t)ids % 4 || (uintptr_t)dst % 4)
        return OUTPROD_E_LAYOUT;
    if (n_used > 1 && nb[13] < 4 * ne00) return OUTPROD_E_LAYOUT;
    if (n_tok > 1 && nb[14] < (n_used - 1) * nb[13] + 4 * ne00) return OUTPROD_E_LAYOUT;
    if (!dst) return OUTPROD_E_NULL;
    if (K > 0 && (!as || !g || !ids)) return OUTPROD_E_NULL;

    // index range (32-bit kernel indices) and extents
    const int64_t lim = INT32_MAX;
    if (ne00 > lim || K > lim || slots > lim / 4 || E > kIdMaxExperts) return OUTPROD_E_RANGE;
    const int64_t a_row = ne00 / block_values(as_type) * block_bytes(as_type);
    int64_t ext_a = 0, ext_g = 0, ext_i = 0, ext_d = 0;
    {
        const int64_t dne[4] = {ne00, n_used, n_tok, 1}, dnb[4] = {4, nb[13], nb[14], nb[15]};
        if (!extent(4 * ne00, dne, dnb, &ext_d)) return OUTPROD_E_RANGE;
    }
    if (K > 0) {
        const int64_t ane[4] = {ne00, K, E, 1}, anb[4] = {nb[0], nb[1], nb[2], nb[3]};
        const int64_t gne[4] = {K, n_used, n_tok, 1}, gnb[4] = {4, nb[5], nb[6], nb[7]};
        const int64_t ine[4] = {n_used, n_tok, 1, 1}, inb[4] = {4, nb[9], nb[10], nb[11]};
        if (!extent(a_row, ane, anb, &ext_a) || !extent(4 * K, gne, gnb, &ext_g) ||
            !extent(4 * n_used, ine, inb, &ext_i))
            return OUTPROD_E_RANGE;
        if (overlaps(dst, ext_d, as, ext_a) || overlaps(dst, ext_d, g, ext_g) ||
            overlaps(dst, ext_d, ids, ext_i))
            return OUTPROD_E_ALIAS;
    }

    p.as = (const uint8_t *)as;
    p.g = (const uint8_t *)g;
    p.ids = (const uint8_t *)ids;
    p.dst = (uint8_t *)dst;
    p.nb01 = nb[1];
    p.nb02 = nb[2];
    p.nbg1 = nb[5];
    p.nbg2 = nb[6];
    p.nbi1 = nb[9];
    p.nbd1 = nb[13];
    p.nbd2 = nb[14];
    p.vec_a = (as_type == OUTPROD_TYPE_F32 || as_type == OUTPROD_TYPE_F16 ||
               as_type == OUTPROD_TYPE_BF16) &&
              (uintptr_t)as % 16 == 0 && nb[1] % 16 == 0 && nb[2] % 16 == 0;
    p.vec_g = (uintptr_t)g % 16 == 0 && nb[5] % 16 == 0 && nb[6] % 16 == 0;

    const int fam = kernel & 0xFF, variant = (kernel >> 8) & 0xFF;
    if ((kernel >> 16) != 0 || (fam != OUTPROD_KERNEL_AUTO && fam != OUTPROD_KERNEL_TILED))
        return OUTPROD_E_KERNEL;
    if (K == 0) {
        c->zero = true;
        l.kernel = OUTPROD_KERNEL_ZERO;
        return OUTPROD_OK;
    }
    l.variant = variant;
    if (!plan_id_back(p, &l)) return OUTPROD_E_KERNEL;
    if (l.grid > lim || id_workspace_bytes(p) > kWorkspaceBytes) return OUTPROD_E_RANGE;
    return OUTPROD_OK;
}

// dst rows of an ID problem as an OUT_PROD dst (for the zero kernel)
Problem id_dst_as_problem(const IdProblem &q) {
    Problem p;
    memset(&p, 0, sizeof(p));
    p.dst = q.dst;
    p.M = q.M;
    p.N = q.n_used;
    p.ne12 = q.n_tokens;
    p.ne13 = 1;
    p.nb0 = 4;
    p.nb1 = q.nbd1;
    p.nb2 = q.nbd2;
    p.nb3 = 0;
    p.dps2 = p.dps3 = 1;
    return p;
}

int run_id_back(const void *as, int as_type, const float *g, const int32_t *ids, float *dst,
                const int64_t *ne, const int64_t *nb, void *stream, int kernel) {
    IdChecked c;
    int rc = validate_id_back(as, as_type, g, ids, dst, ne, nb, kernel, &c);
    if (rc != OUTPROD_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (c.l.kernel == OUTPROD_KERNEL_NONE) return OUTPROD_OK;
    hipError_t e;
    if (c.zero) {
        Problem z = id_dst_as_problem(c.p);
        Launch zl;
        memset(&zl, 0, sizeof(zl));
        plan_zero(z, &zl);
        e = launch_zero(z, zl, s);
    } else {
        uint8_t *ws = nullptr;
        rc = stream_workspace(s, &ws);
        if (rc != OUTPROD_OK) return rc;
        c.p.ws = ws;
        e = launch_id_back(c.p, c.l, s);
    }
    return e == hipSuccess ? OUTPROD_OK : OUTPROD_E_HIP;
}

}  // namespace
}  // namespace outprod

extern "C" {

int out_prod_id_back(const void *as, int as_type, const float *g, const int32_t *ids, float *dst,
                     const int64_t ne[16], const int64_t nb[16], void *stream) {
    return outprod::run_id_back(as, as_type, g, ids, dst, ne, nb, stream, OUTPROD_KERNEL_AUTO);
}

int out_prod_id_back_ex(const void *as, int as_type, const float *g, const int32_t *ids, float *dst,
                        const int64_t ne[16], const int64_t nb[16], void *stream, int kernel) {
    return outprod::run_id_back(as, as_type, g, ids, dst, ne, nb, stream, kernel);
}

int out_prod_id_back_plan(const void *as, int as_type, const float *g, const int32_t *ids,
                          const float *dst, const int64_t ne[16], const int64_t nb[16], int kernel,
                          outprod_plan *plan) {
    if (!plan) return OUTPROD_E_NULL;
    outprod::IdChecked c;
    int rc = outprod::validate_id_back(as, as_type, g, ids, dst, ne, nb, kernel, &c);
    if (rc != OUTPROD_OK) return rc;
    memset(plan, 0, sizeof(*plan));
    plan->kernel = c.l.kernel;
    plan->tile_m = c.l.tile_m;
    plan->tile_n = c.l.tile_n;
    plan->tile_k = c.l.tile_k;
    plan->block = c.l.block;
    plan->lds_bytes = c.l.lds_bytes;
    plan->grid = c.l.grid;
    plan->slices = c.p.n_used * c.p.n_tokens;
    plan->dps2 = plan->dps3 = 1;
    plan->flops = 2 * c.p.M * c.p.K * c.p.n_used * c.p.n_tokens;
    plan->variant = c.l.variant;
    plan->splits = 1;
    plan->ksplit = c.p.K;
    plan->workspace_bytes = c.l.kernel == OUTPROD_KERNEL_TILED ? outprod::id_workspace_bytes(c.p) : 0;
    plan->group_m = 0;
    return OUTPROD_OK;
}


int out_prod(const void *a, int a_type, const float *b, float *dst, const int64_t ne[12],
             const int64_t nb[12], void *stream) {
    return outprod::run(a, a_type, b, dst, ne, nb, stream, OUTPROD_KERNEL_AUTO);
}

int out_prod_ex(const void *a, int a_type, const float *b, float *dst, const int64_t ne[12],
                const int64_t nb[12], void *stream, int kernel) {
    return outprod::run(a, a_type, b, dst, ne, nb, stream, kernel);
}

int out_prod_plan(const void *a, int a_type, const float *b, const float *dst,
                  const int64_t ne[12], const int64_t nb[12], int kernel, outprod_plan *plan) {
    if (!plan) return OUTPROD_E_NULL;
    outprod::Checked c;
    int rc = outprod::validate_and_plan(a, a_type, b, dst, ne, nb, kernel, &c);
    if (rc != OUTPROD_OK) return rc;
    memset(plan, 0, sizeof(*plan));
    plan->kernel = c.l.kernel;
    plan->tile_m = c.l.tile_m;
    plan->tile_n = c.l.tile_n;
    plan->tile_k = c.l.tile_k;
    plan->block = c.l.block;
    plan->lds_bytes = c.l.lds_bytes;
    plan->grid = c.l.grid;
    plan->slices = c.p.ne12 * c.p.ne13;
    plan->dps2 = c.p.dps2;
    plan->dps3 = c.p.dps3;
    plan->flops = 2 * c.p.M * c.p.N * c.p.K * plan->slices;
    plan->variant = c.l.variant;
    plan->swapped = c.swapped ? 1 : 0;
    plan->splits = c.l.splits > 1 ? c.l.splits : 1;
    plan->ksplit = c.l.splits > 1 ? c.l.ksplit : c.p.K;
    plan->workspace_bytes = outprod::split_bytes(c.p, plan->splits);
    plan->group_m = c.l.kernel == OUTPROD_KERNEL_TILED ? c.l.group_m : 0;
    return OUTPROD_OK;
}

int out_prod_release_stream(void *stream) {
    return outprod::release_stream((hipStream_t)stream);
}

int out_prod_workspace_count(int *count) {
    if (!count) return OUTPROD_E_NULL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return OUTPROD_E_HIP;
    std::lock_guard<std::mutex> lock(outprod::g_ws_mutex);
    *count = 0;
    for (const outprod::Workspace &w : outprod::g_ws)
        if (w.device == dev) ++*count;
    return OUTPROD_OK;
}

const char *out_prod_strerror(int status) {
    switch (status) {
    case OUTPROD_OK: return "success";
    case OUTPROD_E_NULL: return "NULL pointer where memory is required";
    case OUTPROD_E_TYPE: return "unsupported a_type (not one of the OUTPROD_TYPE_* ids)";
    case OUTPROD_E_SHAPE: return "negative extent";
    case OUTPROD_E_K: return "a.ne[1] != b.ne[1] (contraction length mismatch)";
    case OUTPROD_E_DST_SHAPE: return "dst shape is not {a.ne0, b.ne0, b.ne2, b.ne3}";
    case OUTPROD_E_BCAST: return "b.ne2/b.ne3 not divisible by a.ne2/a.ne3";
    case OUTPROD_E_QK: return "quantized a width is not a whole number of blocks";
    case OUTPROD_E_LAYOUT: return "unsupported strides, alignment or overlapping dst dims";
    case OUTPROD_E_ALIAS: return "dst overlaps an input";
    case OUTPROD_E_RANGE: return "extent exceeds the supported index range";
    case OUTPROD_E_KERNEL: return "the requested kernel cannot run this problem";
    case OUTPROD_E_HIP: return "a HIP call failed (kernel launch or workspace allocation)";
    case OUTPROD_E_CAPTURE:
        return "the call needs a workspace, the stream is capturing a graph and has none "
               "bound (or a release under capture): make one uncaptured call on this stream first";
    case OUTPROD_E_SCRATCH:
        return "the plan's split partials exceed out_prod_noalloc's 32 MiB static scratch";
    case OUTPROD_E_WORKSPACE:
        return "the device's workspaces (4) are all bound to other streams: release a stream "
               "that no longer needs one with out_prod_release_stream";
    default: return "unknown status";
    }
}

int out_prod_version(void) { return 3; }

}  // extern "C"
