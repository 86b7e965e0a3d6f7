/*
 * outprod.h -- C ABI of liboutprod.so: ggml's OUT_PROD on an MI355X (gfx950).
 *
 * The operation (pages: "metal: OUT_PROD runs batched, broadcast and narrow
 * shapes on the GPU", body and review "VERIFIED BY READING"; "metal: OUT_PROD
 * multiplies in float staging", body):
 *
 *   dst[i0,i1,i2,i3] = sum_{k<K} a[i0,k,i2/dps2,i3/dps3] * b[i1,k,i2,i3]
 *   dps2 = ne12/ne02,  dps3 = ne13/ne03          (integer division)
 *
 * It is the whole matmul backward of a training graph: the gradient of a
 * weight is out_prod(activation, grad) and the gradient of an input is
 * out_prod(weight, grad^T).  dst has the shape {a.ne0, b.ne0, b.ne2, b.ne3};
 * a's slice dims must divide b's (grouped-head broadcast: consecutive dst
 * slices share one a slice).  a may be f32, f16 or bf16 of any width, or a
 * frozen quantized weight (q4_0, q4_1, q5_0, q5_1, q8_0, q2_K..q6_K) of
 * whole blocks that is dequantized to f32 in registers.
 * b and dst are f32.  Every value is staged and accumulated in fp32; nothing
 * passes through half precision (training gradients exceed half's 65504).
 *
 * Tensor description (ggml convention, dim 0 fastest):
 *   ne[12] = { a.ne[0..3], b.ne[0..3], dst.ne[0..3] }   element counts
 *            a = [ne00, K, ne02, ne03], b = [ne10, K, ne12, ne13],
 *            dst = [ne00, ne10, ne12, ne13]
 *   nb[12] = byte strides in the same order.
 *     nb[0]: the element or block size of a in bytes (4 for f32, 2 for f16
 *            and bf16, 34 for q8_0, 144 for q4_K, ...: see the type list);
 *            nb[8] must be 4 (dst dim 0 is contiguous).
 *     b: either nb[4] == 4 (row-major: each k selects a contiguous row of ne10
 *            floats) or nb[5] == 4 (K contiguous: a transposed view such as
 *            the grad^T that the matmul backward passes for the input gradient);
 *            the other b stride is any multiple of 4.
 *     nb[1..3], nb[5..7], nb[9..11]: any non-negative byte strides (views,
 *            padded rows, stride-0 broadcast of inputs), aligned to 4 bytes;
 *            a's strides and pointer need only 2-byte alignment for f16,
 *            bf16 and the block types whose size is not a multiple of 4
 *            (q4_0, q5_0, q8_0, q3_K, q6_K).  dst's dims must be ordered and
 *            must not overlap.
 *
 * Memory and ownership: a, b and dst are DEVICE pointers owned by the caller.
 * The library keeps no pointer to them after a call returns.  A call only
 * enqueues work on `stream` (a hipStream_t; NULL = the default stream) and
 * returns; the buffers must stay alive until the stream has passed it.
 * dst is overwritten (not accumulated into).
 *
 * Split K and the workspace: when a problem has too few output tiles to fill
 * the GPU but a long K, the library splits K into ranges (outprod_plan.splits)
 * that run in parallel and write partial results to a workspace; a second
 * kernel on the same stream adds the partials in range order into dst.
 * MUL_MAT_ID_BACK keeps its routing tables in a workspace too.  Workspaces
 * (64 MiB each) belong to the library, at most 4 per device, each bound to
 * one stream, so the library holds at most 256 MiB per device:
 *   - A stream's first call that needs a workspace allocates one (hipMalloc)
 *     and binds it to the stream.  It stays bound until
 *     out_prod_release_stream frees it, so a graph captured on the stream
 *     keeps a valid address.
 *   - Calls on one stream are ordered by the stream; calls on different
 *     streams use different workspaces and may overlap.  A HIP graph keeps
 *     using the workspace of the stream it was captured on: do not replay it
 *     concurrently with calls on that stream or with another replay of a
 *     graph captured there, and do not release that stream while the graph
 *     may still be replayed.
 *   - When a splitting out_prod finds no workspace for its stream (4 are
 *     bound to other streams, or the stream is capturing and has none), it
 *     runs the unsplit plan instead: the same sum in another order, slower
 *     for these shapes, within the same accuracy.  A forced split
 *     (out_prod_ex) returns OUTPROD_E_WORKSPACE or OUTPROD_E_CAPTURE instead,
 *     and so does out_prod_id_back, which has no workspace-free plan.
 * Results are deterministic for a given plan: every dst element has one
 * writer and a fixed summation order, also when K is split.  The plan
 * depends on the problem only, except for the fallback just described.
 * The library's only mutable state is the pool's table, guarded by a mutex;
 * calls may come from any thread.
 *
 * Errors: every function returns OUTPROD_OK (0) or a negative status.  All
 * argument checks happen on the host before any HIP call, and on error dst
 * is left untouched.  Checks run in this order: NULL ne/nb, a_type,
 * negative extents, K mismatch, dst shape, (empty dst: success, no work),
 * broadcast divisibility, quant block width, strides/alignment, NULL data
 * pointers, index range, aliasing, kernel override.
 */
#ifndef OUTPROD_H
#define OUTPROD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* a_type: the GGUF tensor type ids (the frozen-weight types OUT_PROD reads;
 * pages: the MUL_MAT_ID_BACK page's list of out_prod's set).  Block layouts
 * are the GGUF formats, multi-byte fields little-endian; every value is
 * decoded to fp32 in registers, exactly up to one rounding of the block
 * formula.  Bytes per block / values per block: */
#define OUTPROD_TYPE_F32 0   /*   4 / 1 */
#define OUTPROD_TYPE_F16 1   /*   2 / 1: IEEE binary16 */
#define OUTPROD_TYPE_Q4_0 2  /*  18 / 32: fp16 d, 16 bytes of 4-bit q; d*(q-8) */
#define OUTPROD_TYPE_Q4_1 3  /*  20 / 32: fp16 d, fp16 m, 16 bytes of 4-bit q; d*q + m */
#define OUTPROD_TYPE_Q5_0 6  /*  22 / 32: fp16 d, 32 high bits, 16 bytes of nibbles; d*(q-16) */
#define OUTPROD_TYPE_Q5_1 7  /*  24 / 32: fp16 d, fp16 m, 32 high bits, nibbles; d*q + m */
#define OUTPROD_TYPE_Q8_0 8  /*  34 / 32: fp16 d, int8 q[32]; d*q */
#define OUTPROD_TYPE_Q2_K 10 /*  84 / 256: 16 (scale, min) nibble pairs, 2-bit q, fp16 d,
                                 fp16 dmin; d*scale*q - dmin*min */
#define OUTPROD_TYPE_Q3_K 11 /* 110 / 256: high-bit mask, 2-bit low parts, 16 6-bit scales,
                                 fp16 d; d*(scale-32)*q, q in [-4, 3] */
#define OUTPROD_TYPE_Q4_K 12 /* 144 / 256: fp16 d, fp16 dmin, 12 bytes of 6-bit (scale, min)
                                 for 8 sub-blocks of 32, 128 bytes of 4-bit q;
                                 d*scale*q - dmin*min */
#define OUTPROD_TYPE_Q5_K 13 /* 176 / 256: as q4_K plus 32 bytes of high bits; 5-bit q */
#define OUTPROD_TYPE_Q6_K 14 /* 210 / 256: 4-bit low parts, 2-bit high parts, 16 int8
                                 scales, fp16 d; d*scale*(q-32) */
#define OUTPROD_TYPE_BF16 30 /*   2 / 1: the top half of an IEEE binary32 */

/* status codes */
#define OUTPROD_OK 0
#define OUTPROD_E_NULL (-1)      /* ne/nb NULL, or a data pointer NULL where data is read/written */
#define OUTPROD_E_TYPE (-2)      /* a_type is not one of the OUTPROD_TYPE_* ids */
#define OUTPROD_E_SHAPE (-3)     /* a negative extent */
#define OUTPROD_E_K (-4)         /* a.ne[1] != b.ne[1] */
#define OUTPROD_E_DST_SHAPE (-5) /* dst.ne != {a.ne0, b.ne0, b.ne2, b.ne3} */
#define OUTPROD_E_BCAST (-6)     /* b.ne2 % a.ne2 or b.ne3 % a.ne3 != 0 (or a.ne2/a.ne3 < 1) */
#define OUTPROD_E_QK (-7)        /* quantized a whose width is not a whole number of blocks */
#define OUTPROD_E_LAYOUT (-8)    /* bad nb[0], negative or misaligned stride or pointer,
                                    overlapping dst dims */
#define OUTPROD_E_ALIAS (-9)     /* dst's bytes overlap a's or b's */
#define OUTPROD_E_RANGE (-10)    /* an extent overflows the kernels' index range */
#define OUTPROD_E_KERNEL (-11)   /* a forced kernel that cannot run this problem */
#define OUTPROD_E_HIP (-12)      /* a HIP call failed: kernel launch (e.g. no gfx950
                                    device) or the workspace allocation */
#define OUTPROD_E_CAPTURE (-13)  /* the call needs a workspace and the stream is capturing
                                    a graph and has none (see "Split K" above); or a
                                    release under capture */
#define OUTPROD_E_WORKSPACE (-14) /* the call needs a workspace and the device's 4 are
                                     bound to other streams */
#define OUTPROD_E_SCRATCH (-15)  /* out_prod_noalloc: the plan's split partials exceed the
                                    32 MiB static scratch */

/*
 * out_prod: dst = OUT_PROD(a, b) as defined above, enqueued on `stream`.
 * a: device pointer to a's first byte (f32 values or packed blocks).
 * b: device pointer to b's first float.  dst: device pointer to dst's first
 * float.  ne/nb: host arrays of 12 int64 each (read during the call only).
 * K == 0 writes zeros; an empty dst returns OUTPROD_OK without launching.
 */
int out_prod(const void *a, int a_type, const float *b, float *dst,
             const int64_t ne[12], const int64_t nb[12], void *stream);

/* Kernel families (for out_prod_plan's report and out_prod_ex's override). */
#define OUTPROD_KERNEL_AUTO 0   /* let the library choose */
#define OUTPROD_KERNEL_SKINNY 1 /* f32 a only: MFMA column kernels (16x16x4, or 16-block
                                   4x4x1 for narrow a) over strips of 16-64 b columns, K
                                   spread over the waves of a workgroup (and over workgroups
                                   when split); chosen for ne00 <= 32 (bandwidth-bound rank-r
                                   gradients), for a narrow f32 b (operand swap) and for f32
                                   problems with too few output tiles for the tiled kernel */
#define OUTPROD_KERNEL_TILED 2  /* LDS-staged fp32 tiles, MFMA 32x32x2 or 16x16x4, any a
                                   type and shape; a menu of tile configurations (0-14, and
                                   19-20: 272 x 128 tiles whose loads and decode run on 8
                                   waves of their own) */
#define OUTPROD_KERNEL_ZERO 3   /* K == 0: writes zeros */
#define OUTPROD_KERNEL_NONE 4   /* empty dst: nothing to do */

/* What a call would launch.  Filled by out_prod_plan (host only). */
typedef struct outprod_plan {
    int kernel;       /* OUTPROD_KERNEL_* */
    int tile_m;       /* dst tile along i0 (ne00) */
    int tile_n;       /* dst tile along i1 (ne10) */
    int tile_k;       /* K rows per pipeline stage (tiled) or per wave step (skinny) */
    int block;        /* threads per workgroup */
    int lds_bytes;    /* static LDS per workgroup */
    int64_t grid;     /* workgroups in the single launch */
    int64_t slices;   /* ne12 * ne13 */
    int64_t dps2;     /* ne12 / ne02 */
    int64_t dps3;     /* ne13 / ne03 */
    int64_t flops;    /* 2 * ne00 * ne10 * K * slices */
    int variant;      /* configuration index within the family */
    int swapped;      /* 1: run as the operand-swapped problem (narrow f32 b with a
                         wide f32 a); tile_m then runs along ne10, tile_n along ne00 */
    int splits;       /* K ranges run in parallel (1: no split, no reduce kernel) */
    int64_t ksplit;   /* K rows per range (the last range may be shorter) */
    int64_t workspace_bytes; /* partial results: splits * ne00 * ne10 * slices * 4
                                (0 without a split); at most 64 MiB */
    int group_m;      /* tiled kernel: consecutive workgroups walk the tiles of a
                         slice in groups of group_m tiles along i0 (i0 fastest
                         within a group, then i1): tiles along i0 = i0 fastest,
                         1 = i1 fastest; 0 for other kernels */
    int reserved;     /* 0 */
} outprod_plan;

/*
 * out_prod_plan: run every check of out_prod and describe the launch it
 * would make with `kernel` (OUTPROD_KERNEL_AUTO for the library's choice),
 * without touching the device or any HIP API.  The data pointers are only
 * checked (NULL, alignment, aliasing), never dereferenced.  plan must be
 * non-NULL (else OUTPROD_E_NULL).
 */
int out_prod_plan(const void *a, int a_type, const float *b, const float *dst,
                  const int64_t ne[12], const int64_t nb[12], int kernel,
                  outprod_plan *plan);

/*
 * out_prod_ex: out_prod with the kernel family forced (OUTPROD_KERNEL_AUTO,
 * _SKINNY or _TILED), for A/B measurements and for testing both kernels on
 * the same problem.  Bits 8-15 of `kernel` may force a configuration of the
 * family: (index + 1) << 8, with the index as reported in
 * outprod_plan.variant; 0 lets the library choose.  Bits 16-23 may force
 * the split count of K (with a forced family only): 1 = no split, n = n
 * ranges of ceil(K/n) rows (fewer when K is short); 0 lets the library
 * choose.  Bits 24-30 may force the tiled kernel's tile order (with the
 * TILED family only): group_m << 24, 1 <= group_m <= 127 (larger than the
 * tiles along i0 means i0 fastest), as reported in outprod_plan.group_m; 0
 * lets the library choose.  A family, configuration, split or order that
 * cannot run the problem returns OUTPROD_E_KERNEL (e.g. SKINNY for a
 * quantized a, an unknown configuration index -- the tiled family's are
 * 0-14 and 19-20 --, more ranges than K rows, partials beyond the workspace,
 * an order with another family).
 */
int out_prod_ex(const void *a, int a_type, const float *b, float *dst,
                const int64_t ne[12], const int64_t nb[12], void *stream, int kernel);

/*
 * out_prod_id_back: MUL_MAT_ID_BACK, the input gradient of MUL_MAT_ID through
 * frozen experts (pages: the MUL_MAT_ID_BACK Metal-kernel page: one writer per
 * element of a routed slot's row, the expert's rows walked, every type of
 * out_prod's a decoded in registers).  For every routed slot (i, t), i <
 * n_used, t < n_tokens, with e = ids[i, t]:
 *
 *   dst[c, i, t] = sum_{r<K} as[c, r, e] * g[r, i, t]        (c < ne00)
 *
 * i.e. the slot's gradient row times expert e, each expert stored as OUT_PROD
 * stores a (K rows of ne00 values).  dst is per slot; where the forward
 * broadcast one input row to all used experts the caller sums dst over i.
 *
 * ne[16] / nb[16] (ggml order, byte strides), in this order:
 *   as  {ne00, K, n_expert, 1}   nb[0] = element or block bytes of as_type
 *   g   {K, n_used, n_tokens, 1} nb[4] = 4 (K contiguous, f32)
 *   ids {n_used, n_tokens, 1, 1} nb[8] = 4 (int32)
 *   dst {ne00, n_used, n_tokens, 1} nb[12] = 4; rows ordered and disjoint
 * Alignment as for out_prod (a's rules for as; 4 bytes elsewhere).  At most
 * 512 experts.  All pointers are device pointers owned by the caller.
 *
 * The slots are grouped by expert on the device (one routing kernel up to
 * 16384 slots, three beyond; tables in the stream's workspace -- see "Split K
 * and the workspace" above, including OUTPROD_E_CAPTURE and
 * OUTPROD_E_WORKSPACE), then one tiled launch runs every expert's slots: 2 or
 * 4 launches on `stream`.  A slot whose id is outside [0, n_expert) gets a row
 * of NaN (ids are device data; there is no host-side check).  K == 0 writes
 * zeros without reading ids; no slots or ne00 == 0: no work.  Deterministic:
 * each dst row has one writer and sums over K in a fixed order, whichever
 * tile holds its slot (the one-kernel routing orders an expert's slots with
 * atomics, the three-kernel routing keeps their order).  Returns OUTPROD_OK
 * or a status (checks as for out_prod).
 */
int out_prod_id_back(const void *as, int as_type, const float *g, const int32_t *ids, float *dst,
                     const int64_t ne[16], const int64_t nb[16], void *stream);

/* out_prod_id_back with a forced tile configuration: kernel = OUTPROD_KERNEL_TILED
 * | (index + 1) << 8 with an index the grouped kernel is built for (0, 1, 2, 4,
 * 8, 10, 11, 12, 13, and 15-18: slot tiles of 128, 128, 96 and 96 rows built
 * for the grouped kernel only), or OUTPROD_KERNEL_AUTO. */
int out_prod_id_back_ex(const void *as, int as_type, const float *g, const int32_t *ids, float *dst,
                        const int64_t ne[16], const int64_t nb[16], void *stream, int kernel);

/* Every check of out_prod_id_back and the launch it would make (host only):
 * tile sizes, the grid's upper bound (tiles beyond the routed slots' needs exit
 * at once), slots in `slices`, flops, and the workspace bytes. */
int out_prod_id_back_plan(const void *as, int as_type, const float *g, const int32_t *ids,
                          const float *dst, const int64_t ne[16], const int64_t nb[16], int kernel,
                          outprod_plan *plan);

/*
 * out_prod_noalloc: out_prod that allocates nothing, for callers that cannot
 * call hipMalloc -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, checks, plan and result
 * (bit for bit) as out_prod.  A plan that splits K keeps its partials in a
 * 32 MiB scratch array that the library's device image holds on each device
 * (from the first use of the library there until the process ends) instead
 * of a workspace of the pool; a plan whose partials exceed 32 MiB returns
 * OUTPROD_E_SCRATCH before any HIP call, with dst untouched.  Nothing in the
 * scratch needs clearing: a split writes every partial it reads.
 * The first call on a device looks up the scratch's device address
 * (hipGetSymbolAddress); make it outside capture.  Every call on a device
 * shares that device's scratch: splitting calls whose work overlaps on one
 * GPU (other streams, concurrent graph replays) race and must be ordered by
 * the caller.  Calls that do not split K use no scratch.
 */
int out_prod_noalloc(const void *a, int a_type, const float *b, float *dst,
                     const int64_t ne[12], const int64_t nb[12], void *stream);

/*
 * out_prod_release_stream: free the workspace bound to `stream` (a
 * hipStream_t; NULL = the current device's default stream), if any, after
 * waiting for the work queued on `stream` (hipStreamSynchronize).  Call it
 * before destroying a stream that made splitting or MUL_MAT_ID_BACK calls,
 * and only when no graph captured on that stream will be replayed again.
 * It frees device memory, so it must not run while any thread of the process
 * is capturing a graph in global capture mode.  Returns OUTPROD_OK (also
 * when nothing is bound), OUTPROD_E_CAPTURE if `stream` is capturing, or
 * OUTPROD_E_HIP.
 */
int out_prod_release_stream(void *stream);

/*
 * out_prod_workspace_count: how many workspaces the library holds on the
 * current device (at most 4).  OUTPROD_E_NULL for a NULL argument,
 * OUTPROD_E_HIP without a device.
 */
int out_prod_workspace_count(int *count);

/* A static English description of a status code; never NULL. */
const char *out_prod_strerror(int status);

/* Library ABI version: 3 (2 had no group_m in outprod_plan, no workspace
 * pool calls and no out_prod_noalloc; 1 had no split fields). */
int out_prod_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OUTPROD_H */
