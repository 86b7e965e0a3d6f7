// calib.hip -- measurement kernels of libcalib.so (not part of the OUT_PROD
// library): the MI355X's sustained peaks and the read floor of the
// bandwidth-bound shapes, measured on the same device as the kernels they
// are compared with.
//   calib_mfma_f32     a loop of independent v_mfma_f32_32x32x2_f32 (the fp32
//                      matrix-core peak the tiled kernel is held against)
//   calib_read         a grid-stride streaming read (HBM read bandwidth)
//   calib_copy         a grid-stride streaming copy (read + write bandwidth)
//   calib_strip_read   reads a [K][N] fp32 matrix (b's row-major layout) in
//                      strips of `cols` columns and K ranges of `krows` rows,
//                      one workgroup per (strip, range), with every load of a
//                      batch in flight before any use: the least time one
//                      launch needs to move those bytes with that
//                      decomposition (the rank-r gradients' floor)
// Every kernel writes one value per thread (or per element copied) so that
// nothing it loads is dead; all writes stay inside `out`, whose size the
// host wrapper states.
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Each wave runs `iters` rounds of 4 independent 32x32x2 f32 MFMAs (4096
// flops each); out needs gridDim.x * blockDim.x floats.
__global__ __launch_bounds__(256) void mfma_f32_kernel(float *out, int iters) {
    floatx16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
    const float x = 1e-3f * (float)(threadIdx.x & 63);
    const float y = 1.f + 1e-6f * (float)blockIdx.x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[c][j];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Sum of n4 float4 (4 loads per thread per round in flight); out needs
// gridDim.x * blockDim.x floats.
__global__ __launch_bounds__(256) void read_kernel(const floatx4 *src, int64_t n4, float *out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const floatx4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        s += v0 + v1 + v2 + v3;
    }
    for (; i < n4; i += stride) s += src[i];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(256) void copy_kernel(const floatx4 *src, floatx4 *dst, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

// Workgroup g reads strip g % strips (columns [cols*s, cols*s + cols)) of rows
// [krows*r, min(K, krows*r + krows)), r = g / strips.  Lane layout: a row
// segment is cols/4 float4 chunks; thread t takes chunk t % q of row
// t / q + (T/q)*j, U rows per batch with all U loads issued first.  cols is
// a multiple of 4 and at most 4*T; N a multiple of cols; rows 16-byte
// aligned (ld a multiple of 16).  out needs gridDim.x * blockDim.x floats.
template <int U>
__global__ __launch_bounds__(512) void strip_read_kernel(const uint8_t *b, int64_t ld, int K, int strips,
                                                         int cols, int krows, float *out) {
    const int g = blockIdx.x, s = g % strips, r = g / strips;
    const int q = cols / 4;
    const int T = blockDim.x;
    const int rows_per_pass = T / q;
    const int t = threadIdx.x;
    const int chunk = t % q, row0 = t / q;
    const int k0 = r * krows;
    const int k1 = k0 + krows < K ? k0 + krows : K;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (row0 < rows_per_pass) {
        const uint8_t *base = b + (int64_t)s * cols * 4 + (int64_t)chunk * 16;
        int k = k0 + row0;
        for (; k + (U - 1) * rows_per_pass < k1; k += U * rows_per_pass) {
            floatx4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = *(const floatx4 *)(base + (int64_t)(k + u * rows_per_pass) * ld);
#pragma unroll
            for (int u = 0; u < U; ++u) acc += v[u];
        }
        for (; k < k1; k += rows_per_pass) acc += *(const floatx4 *)(base + (int64_t)k * ld);
    }
    out[(int64_t)g * T + t] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

extern "C" {

// grid workgroups of 256 threads; out: grid * 256 floats.
int calib_mfma_f32(float *out, int grid, int iters, void *stream) {
    hipLaunchKernelGGL(mfma_f32_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// src: n4 float4; out: grid * 256 floats.
int calib_read(const void *src, int64_t n4, float *out, int grid, void *stream) {
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const floatx4 *)src, n4, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int calib_copy(const void *src, void *dst, int64_t n4, int grid, void *stream) {
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const floatx4 *)src,
                       (floatx4 *)dst, n4);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// b: [K][N] fp32 rows of ld bytes; strips of cols columns, K ranges of krows
// rows; threads per workgroup (256 or 512); U: 4, 8 or 16 loads in flight per
// thread.  out: strips * ceil(K / krows) * threads floats.  Returns -2 for
// arguments outside the kernel's assumptions.
int calib_strip_read(const void *b, int64_t ld, int K, int N, int cols, int krows, int threads, int U,
                     float *out, void *stream) {
    if (cols < 4 || cols % 4 || N % cols || cols / 4 > threads || ld % 16 || (uintptr_t)b % 16 ||
        (threads != 256 && threads != 512) || krows < 1 || K < 1)
        return -2;
    const int strips = N / cols;
    const int ranges = (K + krows - 1) / krows;
    const dim3 grid(strips * ranges), block(threads);
    hipStream_t s = (hipStream_t)stream;
    switch (U) {
    case 4: hipLaunchKernelGGL(strip_read_kernel<4>, grid, block, 0, s, (const uint8_t *)b, ld, K, strips, cols, krows, out); break;
    case 8: hipLaunchKernelGGL(strip_read_kernel<8>, grid, block, 0, s, (const uint8_t *)b, ld, K, strips, cols, krows, out); break;
    case 16: hipLaunchKernelGGL(strip_read_kernel<16>, grid, block, 0, s, (const uint8_t *)b, ld, K, strips, cols, krows, out); break;
    default: return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
