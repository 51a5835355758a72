/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 group-affine decode library.
 *
 * The operation (letters: M activation rows, N output features, K reduction):
 *
 *     y[m, n] = sum_k x[m, k] * w[n, k],    w[n, k] = q[n, k] * s[n, g] + b[n, g],
 *     g = floor(k / 64)
 *
 * as defined on "Week 2 Day 2: Keep W4 Packed" (tiny-llm book), sections
 * "Group-Wise Affine Quantization", "Reconstruct a Stored Group" (w = q s + b,
 * unsigned 4-bit code, signed scale used as stored) and "Quantized Matrix
 * Multiplication" (C = A B^T with the dequantized B), at the group size 64 of
 * the Gemma-4 megakernel page ("Usage") or the tiny-llm page's 128.  M is 1 for greedy decode or k+1 for
 * a speculative-verify batch (Gemma-4 megakernel page, "What it does": the
 * weights stream once for all M rows).
 *
 * Data layout (all row-major, contiguous, caller-owned DEVICE memory):
 *   x       bf16 bits (uint16_t)  [M][K]
 *   qw      uint32                [N][K/8]   word j of row n holds codes
 *                                            k = 8j .. 8j+7, code 8j+i in bits
 *                                            4i .. 4i+3 ("Packed Storage Layout")
 *   scales  bf16 bits             [N][K/64]
 *   biases  bf16 bits             [N][K/64]
 *   y       bf16 bits or fp32     [M][N]
 *
 * Arithmetic contract: each weight is dequantized as one fp32 fused
 * multiply-add fma(s, q, b) (bit-exact with w4a16_dequant), products are
 * accumulated in fp32 in an order fixed by (N, K) alone, and the bf16 output
 * is the round-to-nearest-even of the fp32 result.  Hence row m of an M-row
 * call is bitwise equal to a 1-row call on x[m] (batch invariance, which the
 * lossless speculative decoding of the Gemma-4 megakernel page relies on).
 *
 * Conventions for every entry point:
 *   - Every pointer is a device pointer owned by the caller; the library
 *     allocates nothing, keeps no state between calls and never synchronizes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); work
 *     is enqueued on it and the call returns immediately.
 *   - Argument errors are detected before anything is enqueued; on any such
 *     error nothing is launched and nothing is written.  W4A16_ERR_HIP (the
 *     runtime refused a launch) is the exception: entry points that enqueue
 *     more than one kernel (w4a16_matmul_grouped, w4a16_lmhead_argmax, the
 *     chunked w4a16_matmul_prefill) may have enqueued the earlier ones, so the
 *     outputs are then unspecified.
 *   - Calls are re-entrant.  Outputs must not alias inputs.
 *   - Empty problems (M == 0 or N == 0) succeed without launching.
 *   - Sizes: 0 <= N <= W4A16_MAX_N and K <= W4A16_MAX_K (so that every block
 *     count and every byte offset inside one wave's rows fits 32 bits);
 *     larger sizes return W4A16_ERR_SHAPE.
 *   - Alignment: qw and x 16 bytes (both are read with 16-byte loads);
 *     scales, biases 2 bytes; y 2 bytes (bf16) or 4 bytes (fp32); ids,
 *     argmax 4 bytes; workspace 8 bytes.
 *   - 4-bit codes with group == 64 (the workload's) or group == 128 (the
 *     tiny-llm page's); K must be a multiple of the group.
 *   - Asynchronous device faults surface at the caller's next synchronization.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 2
#define W4A16_MAX_M 8
#define W4A16_MAX_PREFILL_M 65536
#define W4A16_MAX_GROUP 8
#define W4A16_MAX_N (1 << 30)
#define W4A16_MAX_K (1 << 24)
#define W4A16_NOALLOC_SCRATCH_BYTES (1 << 20)

typedef enum w4a16_status {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,        /* a required pointer is NULL */
    W4A16_ERR_SHAPE = 2,       /* a size is negative, K is not a positive multiple of the
                                  group, N > W4A16_MAX_N, K > W4A16_MAX_K, top_k/E/R or
                                  a stride out of range */
    W4A16_ERR_UNSUPPORTED = 3, /* group not 64 or 128, M above the entry point's maximum,
                                  or an unknown out_dtype */
    W4A16_ERR_ALIGN = 4,       /* a pointer violates the alignment above */
    W4A16_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    W4A16_ERR_HIP = 6,         /* the HIP runtime rejected a launch */
    W4A16_ERR_SCRATCH = 7,     /* a no-allocation entry point's problem needs more than
                                  W4A16_NOALLOC_SCRATCH_BYTES of built-in scratch */
    W4A16_STATUS_MAX_ENUM = 0x7FFFFFFF  /* not a status: gives the type the range of a 32-bit
                                           int, so any value a caller passes back to
                                           w4a16_status_str is a valid value of it */
} w4a16_status_t;

typedef enum w4a16_out {
    W4A16_OUT_BF16 = 0,        /* y holds bf16 bits, round-to-nearest-even of the fp32 sum */
    W4A16_OUT_F32 = 1          /* y holds the fp32 sum itself (same arithmetic) */
} w4a16_out_t;

/*
 * Dense product, 1 <= M <= 8 (qmv at M = 1, skinny qmm at M = 2..8).
 * Definition: "Quantized Matrix Multiplication" / "Computation Flow" on the
 * tiny-llm W4 page, with the group size of the Gemma-4 page (64) or of the
 * tiny-llm page (128).
 * y: [M][N], bf16 or fp32 per out_dtype.
 */
w4a16_status_t w4a16_matmul(const uint16_t *x, const uint32_t *qw, const uint16_t *scales,
                            const uint16_t *biases, void *y, int out_dtype, int M, int N, int K,
                            int group, void *stream);

/*
 * Gated MLP activation on a fused gate+up matrix (the GeGLU MLP of the
 * Gemma-4 megakernel page, "What it does"): qw/scales/biases describe a
 * [2I][K] matrix whose rows 0..I-1 are the gate projection and rows I..2I-1
 * the up projection (the fused gate_up layout), and
 *   h[m][j] = GELU(g) * u,  g = (x W^T)[m][j],  u = (x W^T)[m][I + j],
 * with the exact GELU, GELU(g) = g * Phi(g) (the page names GeGLU but not the
 * GELU form; the exact one is the reading taken).  g and u are bitwise the
 * fp32 sums w4a16_matmul produces for those rows of the same matrix; the
 * activation is computed in fp32 and h rounded once per out_dtype.
 * h: [M][I].  1 <= M <= 8, any I >= 0 (M = 0 or I = 0 writes nothing).
 */
w4a16_status_t w4a16_matmul_geglu(const uint16_t *x, const uint32_t *qw, const uint16_t *scales,
                                  const uint16_t *biases, void *h, int out_dtype, int M, int I,
                                  int K, int group, void *stream);

/*
 * Prefill-shaped product, 1 <= M <= W4A16_MAX_PREFILL_M activation rows (a
 * prompt's tokens): the same y = x W^T and dequantization as w4a16_matmul,
 * computed on the matrix cores (tiny-llm page, "Revisit the Decode Roofline":
 * prefill reuses each weight across many rows and needs a matrix schedule).
 * Up to 16 rows run the decode kernels on chunks of at most 8 rows (each
 * chunk bitwise equal to a w4a16_matmul call on those rows; a launch error
 * on the second chunk leaves the first chunk's rows written).  Larger M with
 * at least 96 output tiles of 128 x 128 (and M > 64), or 160..255 of
 * 64 x 128 (and M > 40), use the page's rearranged sums ("Quantized Matrix
 * Multiplication"): per 64 codes,
 * y += s * sum(x * (q - 8)) + (b + 8 s) * sum(x), the centred codes entering
 * the matrix cores as exact bf16 integers; its rounding is bounded on
 * sum |s x (q - 8)| + |(b + 8 s) x| rather than sum |w x| (close for
 * b ~ -8 s; a stored zero weight, q = 8 and b = -8 s, contributes exactly 0).
 * Smaller grids dequantize each weight with fma(s, q, b) and split it into
 * bf16 hi + lo parts (bounded on sum |w x| like w4a16_matmul).  Above 16
 * rows both orders differ from the M <= 8 schedules: no bitwise equality
 * with w4a16_matmul.  Deterministic.  Meant for M > 8.
 * Needs 8 |s| and |s| * 15 finite in fp32.
 */
w4a16_status_t w4a16_matmul_prefill(const uint16_t *x, const uint32_t *qw, const uint16_t *scales,
                                    const uint16_t *biases, void *y, int out_dtype, int M, int N,
                                    int K, int group, void *stream);

/*
 * One matrix of a grouped product: packed weights, scales, biases and its
 * output y [M][N] (bf16 or fp32 per the call's out_dtype).
 */
typedef struct w4a16_matrix {
    const uint32_t *qw;        /* [N][K/8] */
    const uint16_t *scales;    /* [N][K/64] */
    const uint16_t *biases;    /* [N][K/64] */
    void *y;                   /* [M][N] */
    int N;
} w4a16_matrix_t;

/*
 * Grouped product: `count` (<= W4A16_MAX_GROUP) matrices with the same K that
 * multiply the same activations x [M][K], computed in as few launches as the
 * row schedule allows (one for the q, k and v projections of a decode layer).
 * Each output is bitwise equal to a w4a16_matmul call on that matrix alone.
 * This is the fused q/k/v launch the Gemma-4 megakernel page motivates (one
 * launch instead of several for small decode projections, "What it does").
 * `mats` is a HOST array read during the call; every pointer in it is device
 * memory with the alignment of w4a16_matmul.  Matrices with N == 0 are skipped.
 */
w4a16_status_t w4a16_matmul_grouped(const uint16_t *x, const w4a16_matrix_t *mats, int count,
                                    int out_dtype, int M, int K, int group, void *stream);

/*
 * Routed (expert-gathered) product for MoE decode: the routed-expert matvec
 * (mul_mv_id) of the hy4-preview-metal page's kernel table.
 *   qw [E][N][K/8], scales/biases [E][N][K/64]  (expert e = slab e)
 *   ids int32 [M][top_k], each in [0, E)
 *   x   x_slot_stride == 0: [M][K], row m shared by token m's slots;
 *       x_slot_stride >= K: one row per slot, slot (m, j) reading the K
 *       values at x + (m * top_k + j) * x_slot_stride (elements; a multiple
 *       of 8 so that every row keeps the 16-byte alignment; K gives the dense
 *       [M][top_k][K] layout)
 *   y   [M][top_k][N]:  y[m][j][:] = W_{ids[m][j]} . x[m] (or slot (m, j)'s row)
 * Each distinct expert's weights are streamed once for all slots routed to
 * it.  No routing weights are applied.  An id outside [0, E) is a
 * precondition violation: the slot's output row is filled with NaN.
 * 1 <= M <= 8, 1 <= top_k <= 64, 1 <= E; any other x_slot_stride (negative,
 * between 1 and K - 1, not a multiple of 8) returns W4A16_ERR_SHAPE.
 */
w4a16_status_t w4a16_matmul_id(const uint16_t *x, int64_t x_slot_stride, const uint32_t *qw,
                               const uint16_t *scales, const uint16_t *biases, const int32_t *ids,
                               void *y, int out_dtype, int M, int top_k, int E, int N, int K,
                               int group, void *stream);

/*
 * Bytes of device workspace w4a16_lmhead_argmax needs for this shape
 * (0 when the arguments are invalid).
 */
size_t w4a16_lmhead_argmax_workspace_bytes(int M, int N, int K, int group);

/*
 * Tied LM head with fused per-row argmax: the 4-bit vocabulary projection
 * with in-kernel argmax of the Gemma-4 megakernel page ("What it does", draft
 * kernel), the tied output head of the tiny-llm page (Task 1, as_linear).
 *   logits [M][N] (bf16 or fp32 per out_dtype), or NULL to skip writing them
 *   argmax int32 [M]: index of the largest fp32 logit of row m; ties go to the
 *          lowest index; a NaN logit ranks above every number.
 *   workspace: at least w4a16_lmhead_argmax_workspace_bytes(M, N, K, group)
 *          bytes of device memory; its contents need no initialization and
 *          are scratch for this call only.
 * Two kernels run on `stream`: the product with per-block partial argmax,
 * then an ordered finalize.  Deterministic.
 */
w4a16_status_t w4a16_lmhead_argmax(const uint16_t *x, const uint32_t *qw, const uint16_t *scales,
                                   const uint16_t *biases, void *logits, int out_dtype,
                                   int32_t *argmax, void *workspace, size_t workspace_bytes,
                                   int M, int N, int K, int group, void *stream);

/*
 * w4a16_lmhead_argmax without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * w4a16_lmhead_argmax; the per-block argmax keys go to a scratch array built
 * into the library (W4A16_NOALLOC_SCRATCH_BYTES on each GPU, held until the
 * process ends; its device address is looked up on the first call on each
 * device).  Nothing is allocated.  A problem whose workspace
 * (w4a16_lmhead_argmax_workspace_bytes) exceeds the scratch returns
 * W4A16_ERR_SCRATCH before anything is enqueued (1 MiB covers a 262144-row
 * vocabulary at every M).  Every call on one GPU shares that GPU's scratch:
 * calls that overlap in time on one GPU (concurrent streams, or host threads
 * enqueueing onto different streams) race and must be serialized by the
 * caller; calls in order on one stream are safe.  Nothing carries over from
 * one call to the next (every key the finalize reads is written by the same
 * call), so the scratch needs no clearing.
 */
w4a16_status_t w4a16_lmhead_argmax_noalloc(const uint16_t *x, const uint32_t *qw, const uint16_t *scales,
                                           const uint16_t *biases, void *logits, int out_dtype,
                                           int32_t *argmax, int M, int N, int K, int group,
                                           void *stream);

/*
 * Dequantized weights out[r][k] = fma(s, q, b) in fp32 for rows[r] (rows ==
 * NULL: every row, R = N), the same value the products use for each weight
 * ("Reconstruct a Stored Group").  Also the quantized row gather of an
 * embedding lookup (tiny-llm page, Task 1: dequantize selected rows without
 * expanding the table).  A row index outside [0, N) writes NaN to that row.
 * out: fp32 [R][K], 16-byte aligned; qw needs only 4-byte alignment here.
 */
w4a16_status_t w4a16_dequant(const uint32_t *qw, const uint16_t *scales, const uint16_t *biases,
                             const int32_t *rows, int R, float *out, int N, int K, int group,
                             void *stream);

/*
 * Quantized row gather for an embedding lookup: out[r][k] = bf16 round to
 * nearest even of fma(s, q, b), i.e. of w4a16_dequant's value, for the table
 * row n = rows[r] (tiny-llm page, Task 1: the selected rows are dequantized
 * straight from the packed table, which is never expanded; the Gemma-4
 * megakernel page dequantizes its 4-bit embedding inside the kernel).
 * rows: int32 [R] on the device, any order, repeats allowed; a row index
 * outside [0, N) writes bf16 NaN (0x7FC0) to that output row.
 * qw: 4-byte aligned; out: bf16 [R][K], 16-byte aligned.  R == 0 succeeds
 * without launching.
 */
w4a16_status_t w4a16_gather_rows(const uint32_t *qw, const uint16_t *scales, const uint16_t *biases,
                                 const int32_t *rows, int R, uint16_t *out, int N, int K, int group,
                                 void *stream);

/*
 * Packed-weight loader: codes uint8 [N][K] (low 4 bits used) -> qw uint32
 * [N][K/8] in the layout above ("Packed Storage Layout").  K % 8 == 0.
 */
w4a16_status_t w4a16_pack(const uint8_t *codes, uint32_t *qw, int N, int K, void *stream);

/* Static description of a status code (never NULL). */
const char *w4a16_status_str(w4a16_status_t s);

/*
 * Name of the kernel instantiation w4a16_matmul launches for this shape, as
 * profilers report it ("qmm_dense_kernel<M, R, CPL, KSPLIT, PRE, DEPTH, RS, G>":
 * activation rows, rows per lane, 16-byte chunks per lane per K-tile, waves
 * sharing a row, chunk slots whose loads are issued before the activations are
 * staged, chunk slots in flight per lane, row sets per block when KSPLIT > 1,
 * group size).
 * "" when the arguments are invalid.  The string lives in thread-local storage
 * and stays valid until the next call on the same thread.
 */
const char *w4a16_schedule_name(int M, int N, int K, int group);

/* W4A16_ABI_VERSION of the loaded library. */
int w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
