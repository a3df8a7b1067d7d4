/*
 * lora.h -- C ABI of liblora.so: a fused LoRA linear forward and the merge of
 * a LoRA adapter into a pristine copy of the base weight, on AMD Instinct
 * MI355X (gfx950).
 *
 * Definitions (page titles as published):
 *   [fastaf]  "fastaf: Minimal LoRA fine-tuning with hand-written Triton
 *             kernels", section "FWD kernel speedup": one LoRA layer computes
 *             out = X W^T + ((X A^T) B^T) * scale, scale = alpha / r, and the
 *             fused kernel keeps the [tokens, r] intermediate X A^T on chip;
 *             section "BWD kernel speedup": its backward produces dA, dB and
 *             dX, and dA is parallelised over the sequence; section "Block
 *             size tuning": candidate tile configurations are pruned by the
 *             device's per-block thread, register and shared-memory limits
 *             and a minimum occupancy, the survivors benchmarked, and the
 *             winner cached per shape (nearest shape on a miss, else a
 *             default).
 *   [unsloth] unsloth commit log for scripts/benchmarks/qwen3_flex_inference.py,
 *             the entry that replaces copy+merge_adapter by one
 *             addmm(pristine, B, A, alpha=scaling, out=W_inf) per layer: the
 *             pristine weight is only read, W_inf is rewritten, accumulation
 *             is fp32; rsLoRA folds alpha/sqrt(r) into the same scaling.
 *
 * Conventions shared by every entry point:
 *   - Layouts follow nn.Linear: X[M,K] (tokens x d_in), W[N,K] (d_out x d_in),
 *     A[r,K], B[N,r], Y[M,N]; row-major, unit inner stride, leading dimension
 *     (ld*) in elements, ld >= row length.
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no memory and keeps no state between calls; it is reentrant.
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued there and the call returns without synchronising:
 *     LORA_OK means "validated and launched", not "finished".
 *   - Every argument is validated on the host before any HIP call; on error
 *     nothing is launched and nothing is written.
 *   - One element type for all operands and the result (lora_dtype).
 *     Accumulation is fp32; the result is rounded once, to nearest-even.
 *   - LORA_BF16: pointers 16-byte aligned; K and the ld of X, W, A, W0 and
 *     W_inf multiples of 8.  LORA_F32: pointers 16-byte aligned; K and those
 *     ld multiples of 4.  N, r, ldb and ldy are unrestricted.
 *   - Limits (LORA_ERR_UNSUPPORTED beyond them): every size <= 2^30 - 1;
 *     for lora_fwd, ldx, ldw and lda <= LORA_MAX_LD elements (the kernels
 *     address a 256-row tile of X or W with signed 32-bit byte ranges), and
 *     r * lda * (element size) <= 2^31 - 1 (A as one such range; binding
 *     only for fp32 above rank 128).
 *   - Outputs must not overlap any input (LORA_ERR_ALIAS).
 *   - NaN and Inf in the inputs propagate as IEEE arithmetic makes them.
 */
#ifndef LORA_H
#define LORA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 17

typedef enum lora_status {
    LORA_OK = 0,
    LORA_ERR_NULL = 1,        /* a required pointer is NULL */
    LORA_ERR_SHAPE = 2,       /* negative size, or r < 1 */
    LORA_ERR_STRIDE = 3,      /* a leading dimension is smaller than its row */
    LORA_ERR_ALIGN = 4,       /* pointer / K / ld alignment rule broken */
    LORA_ERR_DTYPE = 5,       /* unknown lora_dtype */
    LORA_ERR_ALIAS = 6,       /* an output overlaps an input */
    LORA_ERR_UNSUPPORTED = 7, /* r > LORA_MAX_RANK, a size or ld beyond
                                 the limits below, or a forced variant that
                                 cannot run this shape */
    LORA_ERR_HIP = 8,         /* the HIP runtime reported a launch error */
    LORA_ERR_WORKSPACE = 9,   /* lora_bwd workspace NULL, smaller than
                                 lora_bwd_workspace_size or not 256-B aligned */
    LORA_ERR_SCRATCH = 10     /* more forwards than the static scratch of
                                 lora_fwd_batch_noalloc holds */
} lora_status;

#define LORA_MAX_LD ((1 << 22) - 8)

typedef enum lora_dtype {
    LORA_F32 = 0,
    LORA_BF16 = 1
} lora_dtype;

/* Forward variants.  AUTO picks DECODE for bf16 with M <= LORA_DECODE_AUTO_M
 * and r <= 32, TILED otherwise (for 16 < M <= 64 the tiled kernel's small
 * tiles with loader waves stream W from many workgroups, faster there than
 * the decode kernel).  Forcing one is for tests and measurement. */
typedef enum lora_variant {
    LORA_VARIANT_AUTO = 0,
    LORA_VARIANT_TILED = 1,   /* MFMA-tiled fused forward, any M */
    LORA_VARIANT_DECODE = 2   /* weight-streaming forward, bf16, M <= 64 */
} lora_variant;

#define LORA_MAX_RANK 256
#define LORA_DECODE_MAX_M 64
#define LORA_DECODE_AUTO_M 16

/*
 * lora_fwd -- fused LoRA linear forward   [fastaf], "FWD kernel speedup".
 *
 *   Y[m,n] = round( sum_k X[m,k] W[n,k] + scale * sum_j T[m,j] B[n,j] ),
 *   T[m,j] = sum_k X[m,k] A[j,k]   (kept on chip, never stored to memory).
 *
 *   dtype         LORA_F32 or LORA_BF16 (operands and Y).
 *   M, N, K, r    tokens, d_out, d_in, rank.  M == 0 or N == 0: no-op, LORA_OK.
 *                 K == 0: Y = 0.  1 <= r <= LORA_MAX_RANK.
 *   X, ldx        [M,K] activations.
 *   W, ldw        [N,K] base weight.
 *   A, lda        [r,K] down-projection (lora_A).
 *   B, ldb        [N,r] up-projection (lora_B).
 *   scale         alpha / r (or alpha / sqrt(r) for rsLoRA), used as given.
 *   Y, ldy        [M,N] output, fully overwritten; must not overlap X/W/A/B.
 *   stream        hipStream_t as void*.
 * Returns a lora_status.
 */
int lora_fwd(int dtype, int64_t M, int64_t N, int64_t K, int64_t r,
             const void *X, int64_t ldx, const void *W, int64_t ldw,
             const void *A, int64_t lda, const void *B, int64_t ldb,
             float scale, void *Y, int64_t ldy, void *stream);

/*
 * lora_fwd_variant -- lora_fwd with an explicit kernel choice (lora_variant).
 * Same arguments, layouts and errors as lora_fwd; DECODE with dtype != bf16 or
 * M > LORA_DECODE_MAX_M returns LORA_ERR_UNSUPPORTED.
 */
int lora_fwd_variant(int variant, int dtype, int64_t M, int64_t N, int64_t K, int64_t r,
                     const void *X, int64_t ldx, const void *W, int64_t ldw,
                     const void *A, int64_t lda, const void *B, int64_t ldb,
                     float scale, void *Y, int64_t ldy, void *stream);

/*
 * lora_fwd_batch -- several independent forwards in few launches.
 *   [fastaf], "FWD kernel speedup": on small workloads the launch overhead
 *   outweighs the work; a decode step's projections that read the same
 *   tokens (q, k, v; gate, up) are such workloads.
 *
 * Element t of descs describes one forward exactly as the arguments of
 * lora_fwd do; each Y is bitwise what lora_fwd would write.  Consecutive
 * forwards that lora_fwd would run on the decode kernel (bf16,
 * M <= LORA_DECODE_AUTO_M, r <= 32) with the same M and rank class
 * (r <= 16, or 16 < r <= 32) share launches, up to 24 per launch, their
 * descriptors passed as kernel arguments (nothing is allocated); every other
 * forward is launched as lora_fwd would launch it.  Forwards run
 * concurrently, so every Y must also not overlap any other forward's X, W,
 * A, B or Y (LORA_ERR_ALIAS); inputs may be shared.
 *
 * With a workspace, T = X A^T is computed once per forward (A is then read
 * once instead of once per 16 output columns, and the weight stream reads W
 * alone).  For one-token forwards (M = 1) whose launch has more than 256
 * weight workgroups of 16 output columns, the first workgroups of the same
 * launch compute T into the workspace and set a flag there for each weight
 * workgroup, which streams its W meanwhile and waits for its flag only
 * before the epilogue (forwards with more than 30720 output columns take T
 * from a launch of its own); smaller one-token launches ignore the
 * workspace (with one workgroup per CU or fewer, T's latency would add to
 * the stream's).  For 2 <= M <= 16 a small launch computes T first.  One-token forwards stay bitwise lora_fwd's at every rank (T
 * repeats the one-token kernel's partial sums and the stream adds them in
 * its order); for 2 <= M <= 16 the results are bitwise
 * lora_fwd's for r <= 16 (same partition of K, same summation order), while
 * for 16 < r <= 32 the weight stream keeps four 128-deep K blocks per wave in
 * flight, is partitioned differently and Y differs from lora_fwd's by fp32
 * rounding order only (deterministic all the same).
 *
 *   dtype         LORA_F32 or LORA_BF16, for every forward.
 *   count         number of descriptors, >= 0 (0: no-op).
 *   descs         HOST array of count descriptors, read during the call only.
 *   workspace     NULL, or device scratch of workspace_bytes >=
 *                 lora_fwd_batch_workspace_size(count), 256-byte aligned,
 *                 not overlapping any operand; content ignored on entry
 *                 (each launch's flags carry a value of that launch, and
 *                 every flag is cleared again before the launch ends),
 *                 unspecified on return; calls in flight at the same time
 *                 need separate workspaces.
 *   stream        hipStream_t as void*.
 * Returns a lora_status; on any invalid descriptor nothing is launched.
 */
typedef struct lora_fwd_desc {
    int64_t M, N, K, r;
    const void *X;
    int64_t ldx;
    const void *W;
    int64_t ldw;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    float scale;
    void *Y;
    int64_t ldy;
} lora_fwd_desc;

int lora_fwd_batch(int dtype, int count, const lora_fwd_desc *descs, void *workspace,
                   int64_t workspace_bytes, void *stream);

/* Workspace bytes lora_fwd_batch can use for count forwards (16 KiB each),
 * or -1 for count < 0. */
int64_t lora_fwd_batch_workspace_size(int count);

/*
 * lora_fwd_batch_noalloc -- lora_fwd_batch with its workspace in the
 * library's own static device memory, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing and calls no
 * allocating routine; the caller still passes inputs and outputs.
 *
 * Arguments, validation and results as lora_fwd_batch called with a
 * workspace (each Y bitwise the same), for at most LORA_NOALLOC_MAX_FORWARDS
 * descriptors: more return LORA_ERR_SCRATCH and launch nothing.
 *
 * The scratch is one array of LORA_NOALLOC_MAX_FORWARDS x 16 KiB (1 MiB) per
 * GPU, in the library's device data; each GPU holds it from the library's
 * load until the process ends.  Its device address is looked up on the first
 * call on a device, with that device current.  Every call on a GPU uses the
 * same array and overwrites it, and the kernels read only what the same call
 * wrote, so nothing needs clearing between calls; but calls that overlap in
 * time on one GPU (other streams, other threads) race on the array and must
 * be serialised by the caller.
 *
 *   dtype, count, descs, stream   as for lora_fwd_batch.
 * Returns a lora_status (LORA_ERR_HIP if the scratch's address cannot be
 * obtained).
 */
#define LORA_NOALLOC_MAX_FORWARDS 64
int lora_fwd_batch_noalloc(int dtype, int count, const lora_fwd_desc *descs, void *stream);

/*
 * lora_merge -- merge from pristine   [unsloth], addmm refresh entry.
 *
 *   W_inf[n,k] = round( W0[n,k] + scale * sum_j B[n,j] A[j,k] ),
 *
 * one pass: W0 is read once and never written, W_inf is written once and its
 * previous content never read.  Repeated calls with the same inputs give
 * bitwise-identical W_inf (no atomics, fixed summation order).
 *
 *   dtype         LORA_F32 or LORA_BF16 (all of W0, B, A, W_inf).
 *   N, K, r       d_out, d_in, rank.  N == 0 or K == 0: no-op.  1 <= r <= 256.
 *   W0, ldw0      [N,K] pristine base weight (read only).
 *   B, ldb        [N,r] lora_B.
 *   A, lda        [r,K] lora_A.
 *   scale         the adapter's scaling, used as given.
 *   W_inf, ldwi   [N,K] merged weight; must not overlap W0, B or A.
 *   stream        hipStream_t as void*.
 * Returns a lora_status.
 */
int lora_merge(int dtype, int64_t N, int64_t K, int64_t r,
               const void *W0, int64_t ldw0, const void *B, int64_t ldb,
               const void *A, int64_t lda, float scale,
               void *W_inf, int64_t ldwi, void *stream);

/*
 * lora_merge_batch -- lora_merge for many targets in few launches
 *   (the per-layer, per-target refresh loop of [unsloth], all targets of a
 *   model at once).
 *
 * Element t of descs describes one merge exactly as the arguments of
 * lora_merge do.  The result is bitwise the result of calling lora_merge on
 * each target in turn.  Targets are merged concurrently, so every W_inf must
 * also not overlap any other target's W0, B, A or W_inf (LORA_ERR_ALIAS).
 * bf16 targets of the same padded rank go up to 24 per launch, their
 * descriptors passed as kernel arguments (nothing is allocated); fp32
 * targets are launched one by one.
 *
 *   dtype         LORA_F32 or LORA_BF16, for every target.
 *   count         number of descriptors, >= 0 (0: no-op).
 *   descs         HOST array of count descriptors, read during the call only.
 *   stream        hipStream_t as void*.
 * Returns a lora_status; on any invalid descriptor nothing is launched.
 */
typedef struct lora_merge_desc {
    int64_t N, K, r;
    const void *W0;
    int64_t ldw0;
    const void *B;
    int64_t ldb;
    const void *A;
    int64_t lda;
    float scale;
    void *W_inf;
    int64_t ldwi;
} lora_merge_desc;

int lora_merge_batch(int dtype, int count, const lora_merge_desc *descs, void *stream);

/*
 * lora_merge_inplace -- W = round( W + scale * B A ), in place.
 *   [unsloth], the merge_adapter / unmerge_adapter path that the pristine
 *   refresh replaces: merging into the base weight and subtracting again
 *   (scale -> -scale) does not return the base bit for bit in bf16 (about
 *   one ULP of drift per cycle).  Offered as that negative control and for
 *   callers that merge once and never restore.
 *
 *   dtype, N, K, r, B, ldb, A, lda, scale, stream as for lora_merge.
 *   W, ldw        [N,K] weight, read and overwritten; must not overlap B or A.
 * Returns a lora_status.
 */
int lora_merge_inplace(int dtype, int64_t N, int64_t K, int64_t r,
                       void *W, int64_t ldw, const void *B, int64_t ldb,
                       const void *A, int64_t lda, float scale, void *stream);

/*
 * lora_bwd -- backward of the layer with W frozen   [fastaf], "BWD kernel
 * speedup".
 *
 *   T[m,j]  = sum_k X[m,k] A[j,k]          G[m,j] = sum_n dY[m,n] B[n,j]
 *   dX[m,k] = round( sum_n dY[m,n] W[n,k] + scale * sum_j G[m,j] A[j,k] )
 *   dA[j,k] = round( scale * sum_m G[m,j] X[m,k] )
 *   dB[n,j] = round( scale * sum_m dY[m,n] T[m,j] )
 *
 * T and G are rounded to bf16 once before the token contractions (they are
 * MFMA operands there); everything else accumulates in fp32.  dA and dB are
 * contracted over token ranges whose fp32 partial sums are then added in a
 * fixed order: repeated calls give bitwise-identical results (no atomics).
 *
 *   dtype         LORA_BF16 only (LORA_F32: LORA_ERR_UNSUPPORTED).
 *   M, N, K, r    tokens, d_out, d_in, rank; N and K multiples of 8.
 *                 M == 0: dA = 0 and dB = 0 are written.  1 <= r <= 256, and
 *                 (r padded to 16/32/64/128/256) * (M rounded up to 64)
 *                 <= 2^30 - 64.
 *   X, ldx        [M,K] layer input (the forward's X).
 *   W, ldw        [N,K] base weight; only read for dX (may be NULL when dX is).
 *   A, lda        [r,K] lora_A.       B, ldb   [N,r] lora_B.
 *   dY, lddy      [M,N] gradient of the layer output.
 *   scale         the adapter's scaling, as in the forward.
 *   dX, lddx      [M,K] input gradient, or NULL to skip it (frozen input).
 *   dA, ldda      [r,K] gradient of lora_A.
 *   dB, lddb      [N,r] gradient of lora_B.
 *   workspace     device scratch of workspace_bytes >= lora_bwd_workspace_size,
 *                 256-byte aligned, owned by the caller; its content on entry
 *                 is ignored and on return is unspecified.  Calls in flight at
 *                 the same time need separate workspaces.  It holds a
 *                 transposed copy of W (N * K * 2 bytes), T and G, and fp32
 *                 partial sums of dA and dB over token ranges.
 *   stream        hipStream_t as void*.
 * ldx, lda, ldda, lddy and ldw multiples of 8; X, W, A, dY, dA 16-byte
 * aligned.  Outputs and the workspace must not overlap any input or each
 * other (LORA_ERR_ALIAS).  Returns a lora_status.
 */
int lora_bwd(int dtype, int64_t M, int64_t N, int64_t K, int64_t r,
             const void *X, int64_t ldx, const void *W, int64_t ldw,
             const void *A, int64_t lda, const void *B, int64_t ldb,
             const void *dY, int64_t lddy, float scale,
             void *dX, int64_t lddx, void *dA, int64_t ldda, void *dB, int64_t lddb,
             void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes lora_bwd needs for these sizes (0 is possible), or -1 when
 * dtype or the sizes are not supported.  Depends on the sizes only. */
int64_t lora_bwd_workspace_size(int dtype, int64_t M, int64_t N, int64_t K, int64_t r);

/*
 * Tile configurations of the bf16 tiled forward, for a tuner   [fastaf],
 * "Block size tuning".  lora_fwd's own choice (AUTO) is the built-in default;
 * lora_fwd_tile runs one configuration by id.  An id is instantiated only
 * for the padded ranks whose LDS footprint fits the 160 KiB of a CU.
 *
 *   id  tile       waves  T shared over   ranks
 *   0   64 x 32      4    1 N tile        r <= 32
 *   1   128 x 128    8    1               r <= 256
 *   2   128 x 128    8    2 N tiles       r <= 128
 *   3   128 x 128    8    4 N tiles       r <= 128
 *   4   256 x 256    8    1               r <= 64
 *   5   (retired: 256 x 256 with T shared over 2 N tiles spilled at every
 *       rank; never instantiated, lora_tile_get_info returns UNSUPPORTED)
 *   6   128 x 128    8    1               r <= 128   (three stages)
 *   7   128 x 128   16    1               r <= 64    (three stages, k split)
 *   8   128 x 128   12    1               r <= 128   (three stages, 4 loaders)
 *   9   128 x 256   12    1               r <= 32    (three stages, 4 loaders)
 *  10   64 x 64      8    1               r <= 64    (four stages, 4 loaders)
 *  11   64 x 32      8    1               r <= 64    (four stages, 4 loaders)
 *  12   32 x 32      6    1               r <= 64    (four stages, 4 loaders)
 *  13   256 x 160   12    1               r <= 32    (two stages, 4 loaders)
 *  14   128 x 256    8    8 N tiles       64 < r <= 128 (two stages; T kept
 *                                         unpadded after the ring)
 *  15   256 x 256    8    1               r <= 64    (four 32-deep stages,
 *                                         ping-pong: two groups of four waves
 *                                         alternate between multiplying and
 *                                         reading)
 *  16   64 x 32      8    1               r <= 64    (eight stages, 4 loaders)
 *  17   32 x 32      6    1               r <= 64    (eight stages, 4 loaders)
 *  18   256 x 256    8    1               r <= 64    (two stages; waves 0-3
 *                                         issue all stage loads)
 *  19   256 x 256    8    8 N tiles       32 < r <= 128 (T computed once, in
 *                                         a prologue, and kept in LDS after
 *                                         the ring; stages hold X and W only:
 *                                         two 64-deep for r <= 64, three
 *                                         32-deep above; waves 0-3 load)
 * ("T shared over g N tiles": a workgroup computes g consecutive output
 * tiles of one row block and the down-projection T only once.  Every id
 * but 15 and 19 above rank 64 stages 64 k per stage; the stage counts not given are two.  0 keeps
 * eight stages.  "k split": two groups of eight waves compute the same tile,
 * each from one 32-wide half of every stage, and their sums are added before
 * the up-projection; its results differ from the other ids' in rounding,
 * which all agree bit for bit with each other.  "4 loaders": four of the
 * waves only issue the stage loads, the other eight only multiply.)
 */
#define LORA_TILE_COUNT 20

typedef struct lora_tile_info {
    int32_t tile;        /* id */
    int32_t bm, bn;      /* output tile rows (tokens) x columns */
    int32_t waves;       /* 64-lane waves per workgroup */
    int32_t stages;      /* depth of the LDS stage ring */
    int32_t bk;          /* K per stage */
    int32_t group;       /* N tiles per workgroup sharing T */
    int32_t rank_pad;    /* rank the instantiation is padded to */
    int32_t lds_bytes;   /* dynamic LDS per workgroup */
    int32_t k_split;     /* wave groups sharing each stage's k range (1 or 2) */
} lora_tile_info;

typedef struct lora_tile_usage {
    int32_t vgprs;            /* vector registers per lane (numRegs) */
    int32_t scratch_bytes;    /* per-lane spill memory; > 0 means spills */
    int32_t blocks_per_cu;    /* resident workgroups per CU at lds_bytes */
} lora_tile_usage;

typedef struct lora_device_limits {
    int32_t compute_units;
    int32_t lds_per_block;         /* bytes */
    int32_t lds_per_cu;            /* bytes */
    int32_t regs_per_block;
    int32_t max_threads_per_block;
    int32_t wave_size;
} lora_device_limits;

/* Static description of tile `tile` at rank r (no HIP call).
 * LORA_ERR_UNSUPPORTED: no such id, or not instantiated for this rank;
 * LORA_ERR_SHAPE: r < 1; LORA_ERR_NULL: out is NULL. */
int lora_tile_get_info(int tile, int64_t r, lora_tile_info *out);

/* Register, spill and occupancy figures of tile `tile` at rank r on the
 * current device (hipFuncGetAttributes, hipOccupancyMaxActiveBlocksPerMultiprocessor).
 * Errors as lora_tile_get_info, plus LORA_ERR_HIP. */
int lora_tile_get_usage(int tile, int64_t r, lora_tile_usage *out);

/* Limits of the current device (hipGetDeviceProperties). */
int lora_get_device_limits(lora_device_limits *out);

/* lora_fwd with tile configuration `tile` (bf16 only; same arguments,
 * layouts and errors as lora_fwd; LORA_ERR_UNSUPPORTED for f32, an unknown
 * id or one not instantiated for this rank). */
int lora_fwd_tile(int tile, int dtype, int64_t M, int64_t N, int64_t K, int64_t r,
                  const void *X, int64_t ldx, const void *W, int64_t ldw,
                  const void *A, int64_t lda, const void *B, int64_t ldb,
                  float scale, void *Y, int64_t ldy, void *stream);

/* Static, NUL-terminated description of a lora_status value. */
const char *lora_status_str(int status);

/* LORA_ABI_VERSION of the loaded library. */
int lora_abi_version(void);

/* Variant lora_fwd would run for these sizes (a lora_variant, never AUTO). */
int lora_fwd_pick(int dtype, int64_t M, int64_t N, int64_t K, int64_t r);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H */
