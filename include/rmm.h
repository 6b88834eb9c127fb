/*
 * rmm.h -- C ABI of the MI355X (gfx950) Reduced Matrix Multiplication library.
 *
 * Reduced Matrix Multiplication (RMM), as defined in "Reduced Matrix
 * Multiplication: Input-Adaptive Matrix-Product Reduction for LLM Inference"
 * (arXiv 2608.13426), Sec. 3.2: for Y = A B with activations A (n x d) and a
 * weight or intermediate B (d x m), score every contraction index by the
 * column norm s_j = ||A[:, j]||_2, keep the index set I of the ceil(rho d)
 * largest scores (rho in (0, 1] is the retention ratio) and compute only
 * A[:, I] B[I, :].  Sec. 3.3 applies the same rule per attention head to
 * Q K^T (select on Q's columns, gather the same dimensions of the shared GQA
 * K head, scale by 1/sqrt(d_h) with the full d_h) and to linear/MLP
 * projections.
 *
 * Conventions shared by every entry point
 *  - Pointers named A, B, Y, s, idx, workspace are DEVICE pointers on the
 *    current HIP device; descriptors are HOST pointers read during the call.
 *    The caller owns every buffer; the library keeps no pointer after return.
 *  - Matrices are row-major with leading dimensions in elements.
 *  - bf16 is IEEE binary32 truncated to its upper 16 bits (stored as 2-byte
 *    words); bf16 results are rounded to nearest-even from fp32 accumulators.
 *  - All arguments are checked on the host before anything is enqueued; on
 *    any error nothing is launched and no output is written.
 *  - Work is enqueued on `stream` (0 = the null stream); the calls never
 *    synchronize the host.  Device faults surface at the caller's next sync.
 *  - Selection is deterministic: the same inputs give bit-identical indices,
 *    norms and outputs on every call (no atomics in any reduction).
 *  - Index sets are int32, listed in ascending order.  Among equal scores the
 *    lower index is kept.  Scores are ranked as fp32 values with -0 treated as
 *    +0 and NaN above +Inf (finite inputs are the supported case).
 *  - Outputs must not overlap inputs.  Calls that share a workspace must be
 *    ordered (same stream); concurrent calls need separate workspaces.
 */
#ifndef RMM_H
#define RMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below have int as their underlying type in C++ too, so
 * that any int a C caller passes (an unknown status or dtype code included)
 * is a valid value of the parameter and is refused, not undefined. */
#ifdef __cplusplus
#define RMM_ENUM_INT : int
#else
#define RMM_ENUM_INT
#endif

typedef enum RMM_ENUM_INT {
    RMM_OK = 0,
    RMM_ERR_INVALID_ARG = 1, /* a size, pointer, stride or rho is invalid */
    RMM_ERR_UNSUPPORTED = 2, /* valid request the library cannot run */
    RMM_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    RMM_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} rmm_status_t;

typedef enum RMM_ENUM_INT {
    RMM_F32 = 0,  /* fp32 inputs, fp32 FMA accumulation, fp32 output */
    RMM_BF16 = 1  /* bf16 inputs, fp32 accumulation (MFMA), bf16 output */
} rmm_dtype_t;

/* Run the whole path (norms, selection, gather) even when rho = 1.  Without
 * it rho = 1 takes the shortcut I = [0, d) of Sec. 3.2 (every index kept),
 * which gives the same result. */
#define RMM_FLAG_FULL_PATH 0x1

/*
 * |I| = ceil(rho d)  (Sec. 3.2).  rho*d within 1e-9 relative of an integer is
 * taken as that integer (so 0.07 * 100 gives 7, not 8).  Returns 0 when rho
 * is NaN or outside (0, 1], or d < 1; otherwise a value in [1, d].
 */
int64_t rmm_k(double rho, int64_t d);

/* Static, human-readable name of a status code (never NULL). */
const char *rmm_status_string(rmm_status_t status);

/* Name of the last HIP error this thread saw inside the library ("no error"
 * when none): the detail behind RMM_ERR_HIP. */
const char *rmm_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t rmm_version(void);

/*
 * Column norms s_j = ||A[:, j]||_2 for j < d  (Sec. 3.2 importance score).
 *   A        device, n x d row-major, leading dimension lda >= d, dtype dt
 *   s_out    device, d floats; fp32 sums of squares in a fixed order, then a
 *            correctly rounded sqrt
 *   workspace device scratch of at least rmm_colnorm_workspace_size(dt,n,d)
 *            bytes (may be NULL when that size is 0); contents on entry do
 *            not matter
 * Errors: RMM_ERR_INVALID_ARG for n < 1, d < 1, lda < d, NULL A or s_out, or
 * an unknown dtype; RMM_ERR_WORKSPACE for a short workspace.
 * Summation order: each entry point adds the squares of a column in a fixed
 * order, but rmm_colnorm and rmm_matmul (and rmm_gated_mlp) split the rows
 * into different chunks, so their fp32 norms can differ in the last bits.
 * rmm_select(rmm_colnorm(A)) therefore keeps the same set as rmm_matmul's
 * idx_out whenever the k-th and (k+1)-th largest norms differ by more than
 * fp32 rounding (relative ~1e-6); closer than that, each call is still
 * deterministic, but the two may break the near-tie differently.
 */
size_t rmm_colnorm_workspace_size(rmm_dtype_t dt, int64_t n, int64_t d);
rmm_status_t rmm_colnorm(const void *A, rmm_dtype_t dt, int64_t n, int64_t d, int64_t lda,
                         float *s_out, void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * I = TopK(s, k)  (Sec. 3.2) for `batch` independent score vectors.
 *   s        device, batch x d floats (row b at s + b*d)
 *   idx_out  device, batch x k int32 (row b at idx_out + b*k), ascending
 * Exact: an LDS radix select finds the k-th largest score, then an
 * ascending-index compaction keeps every larger score and the lowest-indexed
 * scores equal to it.
 * Errors: RMM_ERR_INVALID_ARG for batch < 1, d < 1, d > 2^31-1, k < 1,
 * k > d, or NULL pointers.
 */
rmm_status_t rmm_select(const float *s, int64_t batch, int64_t d, int64_t k, int32_t *idx_out,
                        hipStream_t stream);

/*
 * Problem descriptor for rmm_matmul (host memory).
 *   dtype        RMM_BF16 or RMM_F32 (A, B and Y share it)
 *   n, d, m      A is n x d, B is d x m, Y is n x m; d is the contraction axis
 *   lda          >= d
 *   ldb          >= m when transB = 0; >= d when transB = 1
 *   ldy          >= m
 *   transB       0: B is stored d x m row-major (weights as in Y = A B);
 *                1: B is stored as B^T, m x d row-major (keys K for
 *                   S = Q K^T, or nn.Linear weights)
 *   batch        >= 1 independent products; entry b uses
 *                A + b*strideA, B + (b / b_group)*strideB, Y + b*strideY
 *                (strides in elements; b_group > 1 shares one B among
 *                b_group consecutive entries: grouped-query attention)
 *   alpha        Y = alpha * A[:, I] B[I, :] (1/sqrt(d_h) for scores, Sec. 3.3)
 *   flags        RMM_FLAG_* bits
 */
typedef struct {
    rmm_dtype_t dtype;
    int32_t transB;
    int64_t n, d, m;
    int64_t lda, ldb, ldy;
    int64_t batch;
    int64_t strideA, strideB, strideY;
    int64_t b_group;
    float alpha;
    int32_t flags;
} rmm_desc_t;

/* Fill a descriptor for one product with dense leading dimensions. */
void rmm_desc_init(rmm_desc_t *desc, rmm_dtype_t dtype, int64_t n, int64_t d, int64_t m);

/*
 * Bytes of device workspace rmm_matmul needs for (desc, rho); 0 means none.
 * Returns SIZE_MAX when the descriptor or rho is invalid.
 */
size_t rmm_workspace_size(const rmm_desc_t *desc, double rho);

/*
 * Which kernels rmm_matmul would run for (desc, rho), decided on the host
 * from sizes alone (alignment of the eventual pointers is assumed).  Writes
 * info[0] = route (RMM_ROUTE_*), info[1] = reduced-product kernel
 * (RMM_GEMM_*, -1 unless the route is RMM_ROUTE_MFMA), info[2] = number of
 * K splits (1 = none; for the decode route, the GEMV's row splits).  For
 * measurement tools and tests that want to know which kernel a shape takes;
 * no GPU call.  Errors: RMM_ERR_INVALID_ARG for an invalid descriptor or rho
 * or a NULL info.
 */
enum {
    RMM_ROUTE_GENERIC = 0, /* fp32 or unaligned operands: FMA tile kernel */
    RMM_ROUTE_MFMA = 1,    /* bf16 matrix-core product */
    RMM_ROUTE_DECODE = 2   /* bf16 single row (n = 1): gathered GEMV */
};
enum {
    RMM_GEMM_TILE256 = 0, /* 256x256 tiles, both operands staged in LDS */
    RMM_GEMM_TILE128 = 1, /* 128x128 tiles (small or short products) */
    RMM_GEMM_ADIRECT = 2, /* 256x256, A in operand blocks straight to registers */
    RMM_GEMM_STREAM = 3,  /* persistent single-K-step kernel (scores Q K^T) */
    RMM_GEMM_BDMA = 4,    /* as ADIRECT, B rows staged by LDS-DMA loads */
    RMM_GEMM_TDMA = 5,    /* 256x256, rows of A^T (written by the norm pass in
                             place of a pack) and of B staged by LDS-DMA loads */
    RMM_GEMM_GCOL = 6     /* narrow output (m <= 128, the P V product of
                             attention): 128-row tiles, A's kept columns
                             gathered from 64-column windows staged in LDS */
};
rmm_status_t rmm_plan_info(const rmm_desc_t *desc, double rho, int32_t *info);

/*
 * The whole reduced product  (Sec. 3.2, 3.3):
 *   1. s_j = ||A_b[:, j]||_2 for every batch entry b,
 *   2. I_b = TopK(s, k) with k = rmm_k(rho, d),
 *   3. gather A_b[:, I_b] and B_g[I_b, :] (g = b / b_group),
 *   4. Y_b = alpha * A_b[:, I_b] B_g[I_b, :].
 *   A, B, Y   device pointers laid out as the descriptor says
 *   idx_out   device, batch x k int32 (row b at idx_out + b*k), or NULL
 *   workspace device scratch of rmm_workspace_size(desc, rho) bytes,
 *             256-byte aligned (as every hipMalloc block is); any contents
 *             on entry
 * Precision: bf16 inputs are contracted on bf16 MFMA with fp32 accumulation
 * (decode, n = 1: fp32 FMA); fp32 inputs with fp32 FMA.  Each output sums
 * its k terms in a fixed order, so repeated calls are bit-identical.
 * Errors: RMM_ERR_INVALID_ARG for an invalid descriptor, rho, NULL A, B,
 * Y, or a workspace that is not 256-byte aligned; RMM_ERR_WORKSPACE when
 * ws_bytes is too small; RMM_ERR_HIP when a
 * launch fails (outputs may then be partly written).
 */
rmm_status_t rmm_matmul(const rmm_desc_t *desc, const void *A, const void *B, double rho, void *Y,
                        int32_t *idx_out, void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * rmm_matmul for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same four steps, kernels and results, bit for bit, but with no workspace
 * argument.  Its scratch memory is a fixed array of
 * RMM_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * until the process ends; the call itself allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine).
 *   desc, A, B, rho, Y, idx_out, stream   as for rmm_matmul
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or different host threads without ordering) race
 * and give undefined results; calls ordered on one stream are safe.  The
 * array keeps whatever the last call left there; nothing in it needs to
 * start at zero.
 * Errors: as for rmm_matmul, plus RMM_ERR_WORKSPACE when
 * rmm_workspace_size(desc, rho) (for these pointers' alignment) exceeds
 * RMM_NOALLOC_SCRATCH_BYTES, detected before anything is launched, and
 * RMM_ERR_HIP when the array's device address cannot be looked up.
 */
#define RMM_NOALLOC_SCRATCH_BYTES (64u << 20)
rmm_status_t rmm_matmul_noalloc(const rmm_desc_t *desc, const void *A, const void *B, double rho, void *Y,
                                int32_t *idx_out, hipStream_t stream);

/*
 * The reduced product over a caller-supplied kept set: steps 3-4 of
 * rmm_matmul with I given instead of selected.  This is the static variant
 * of the selection (Sec. 4, "Baselines": one subset of feature dimensions
 * fixed, e.g. from the prefill activations, and reused for later calls).
 *   idx      device, batch x k int32 (row b at idx + b*k): the kept indices
 *            of batch entry b, strictly ascending in [0, d).  An entry that
 *            is outside [0, d), or not above every earlier in-range entry of
 *            its row, is dropped: Y is then the product over the remaining
 *            entries (a list that meets the precondition loses nothing)
 *   k        1 <= k <= d
 *   workspace device scratch of rmm_workspace_size_indexed(desc, k) bytes,
 *            256-byte aligned; any contents on entry
 * A, B, Y, the descriptor, precision and the fixed summation order are as
 * for rmm_matmul (the same kept set gives the same Y, bit for bit).
 * Errors: RMM_ERR_INVALID_ARG for an invalid descriptor, NULL A, B, Y or
 * idx, k outside [1, d], idx overlapping Y or the workspace, or a workspace
 * that is not 256-byte aligned; RMM_ERR_WORKSPACE when ws_bytes is too small;
 * RMM_ERR_HIP when a launch fails.  rmm_workspace_size_indexed returns
 * SIZE_MAX for an invalid descriptor or k.
 */
size_t rmm_workspace_size_indexed(const rmm_desc_t *desc, int64_t k);
rmm_status_t rmm_matmul_indexed(const rmm_desc_t *desc, const void *A, const void *B, const int32_t *idx,
                                int64_t k, void *Y, void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * The gated MLP block with RMM on its three projections (App. D.1 (ii),
 * eqs. 3-4): Up and Gate map the model dimension d to the intermediate
 * dimension m and select from x's columns, Down maps m back to d and selects
 * from h's columns, each set from its own input:
 *   I = TopK(||x[:, j]||, ceil(rho_in d)),  h = SiLU(x_I Wg_I) * (x_I Wu_I),
 *   J = TopK(||h[:, j]||, ceil(rho_h m)),   Y = h_J Wd_J.
 * The gate is SiLU(z) = z / (1 + e^-z) (the Llama block the paper
 * evaluates); h is rounded to bf16, and its norms are taken from those
 * bf16 values.  Up and Gate read the same x, so one norm pass and one
 * selection serve both, and one GEMM over their interleaved weights
 * computes h with SwiGLU in its epilogue.
 *
 * rmm_gated_weights prepares that operand once, outside the hot path:
 *   Wg, Wu   device bf16, d x m row-major (transposed = 0), or m x d (the
 *            nn.Linear layout, transposed = 1)
 *   Wgu      device bf16, d x 2m, 16-byte aligned: columns 64c..64c+31 hold
 *            Wg's columns 32c..32c+31 and 64c+32..64c+63 Wu's
 * Errors: RMM_ERR_INVALID_ARG for NULL pointers, d < 1, m not a positive
 * multiple of 32, an unaligned Wgu or more than 2^31 bytes.
 *
 * rmm_gated_mlp:
 *   x        device bf16, n x d row-major (dense)
 *   Wgu      from rmm_gated_weights; Wd device bf16, m x d row-major
 *   Y        device bf16, n x d; h_out (n x m bf16), idx_in_out (ceil(rho_in d)
 *            int32, ascending) and idx_h_out (ceil(rho_h m) int32) may be NULL
 *   workspace rmm_gated_mlp_workspace_size(n, d, m, rho_in, rho_h) bytes,
 *            256-byte aligned
 * Supported: n and d multiples of 8, m a multiple of 32, 2m <= 32768, every
 * pointer 16-byte aligned, each operand under 2^31 bytes; otherwise
 * RMM_ERR_UNSUPPORTED (the size query returns SIZE_MAX).  Other errors as for
 * rmm_matmul.  Outputs are bit-reproducible (fixed summation orders).
 */
rmm_status_t rmm_gated_weights(const void *Wg, const void *Wu, int64_t d, int64_t m, int32_t transposed, void *Wgu,
                               hipStream_t stream);
size_t rmm_gated_mlp_workspace_size(int64_t n, int64_t d, int64_t m, double rho_in, double rho_h);
rmm_status_t rmm_gated_mlp(const void *x, const void *Wgu, const void *Wd, int64_t n, int64_t d, int64_t m,
                           double rho_in, double rho_h, void *Y, void *h_out, int32_t *idx_in_out,
                           int32_t *idx_h_out, void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Single-row decode over 8-bit weights (weight-only quantization, W8A16):
 * the gathered GEMV of the decode route with B stored as 8-bit codes and one
 * fp32 scale per output column, the combination of RMM with low-precision
 * weights that App. B.6 ("Compatibility with INT8 Weight Quantization",
 * Table 14) evaluates and App. B.7 leaves to fused quantized kernels.
 *
 *   I = TopK(|a_j|, k = rmm_k(rho, d))  (Sec. 3.2 with n = 1: s_j = |a_j|)
 *   y[c] = alpha * scale[c] * sum_{t<k} a[I_t] * q[I_t, c]
 *
 * a: 1 x d bf16 (16-byte aligned), d <= 16384.  Bq: d x m codes, rows ldb
 * bytes apart (m, ldb multiples of 16; 16-byte aligned): fmt
 * RMM_WQ_FP8_E4M3 = OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 = NaN),
 * RMM_WQ_INT8 = two's-complement int8.  scale: m fp32, the dequantized
 * weight being q * scale[c].  y: 1 x m bf16 (16-byte aligned), rounded to
 * nearest-even from the fp32 sum; the kept rows are summed in fp32 in a
 * fixed order (bit-reproducible).  idx_out (k int32, ascending) may be NULL.
 * The caller owns every buffer; workspace: rmm_decode_wq_workspace_size
 * bytes, 256-byte aligned (SIZE_MAX there means unsupported sizes).
 * Returns RMM_ERR_INVALID_ARG for null pointers, an unknown fmt, bad sizes
 * or overlapping buffers, RMM_ERR_UNSUPPORTED for sizes or alignments
 * outside the above, RMM_ERR_WORKSPACE for a short workspace.
 */
enum { RMM_WQ_FP8_E4M3 = 0, RMM_WQ_INT8 = 1 };

/*
 * Attention with reduced scores and the softmax fused (Sec. 3.2,
 * "Attention"): for each query head h,
 *   I_h = TopK(||Q_h[:, j]||_2, k = rmm_k(rho, dh))   (feature selection on Q)
 *   O_h = softmax(alpha * Q_h[:, I_h] K_g[:, I_h]^T + M) V_g
 * with alpha = 1/sqrt(dh) (the full head dimension), g = h / (H / Hkv) the
 * grouped-query key/value head, and M the causal mask when causal = 1 (query
 * i, the (Lk - Lq + i)-th position, sees keys 0 .. Lk - Lq + i).  The scores
 * never reach HBM.
 *
 * q: H x Lq x dh, k: Hkv x Lk x dh, v: Hkv x Lk x dv, out: H x Lq x dv, all
 * bf16, contiguous, 16-byte aligned; dh <= 128 and a multiple of 8, dv = 128,
 * H a multiple of Hkv, Lq <= Lk when causal.  idx_out (H x k int32, each row
 * ascending) may be NULL.  The softmax runs in fp32 (running maximum and sum,
 * exponentials in base 2), the probabilities enter the value product rounded
 * to bf16, accumulation is fp32 and O is rounded to nearest-even bf16.  The
 * caller owns every buffer; workspace: rmm_attention_workspace_size bytes,
 * 256-byte aligned (SIZE_MAX there: invalid or unsupported sizes).  Returns
 * RMM_ERR_INVALID_ARG for null pointers, bad sizes, causal with Lq > Lk or
 * overlapping buffers, RMM_ERR_UNSUPPORTED for sizes or alignments outside
 * the above, RMM_ERR_WORKSPACE for a short workspace.
 */
size_t rmm_attention_workspace_size(int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t dh, double rho);
rmm_status_t rmm_attention(const void *q, const void *k, const void *v, int64_t H, int64_t Hkv, int64_t Lq,
                           int64_t Lk, int64_t dh, int64_t dv, double rho, int32_t causal, void *out, int32_t *idx_out,
                           void *workspace, size_t ws_bytes, hipStream_t stream);
size_t rmm_decode_wq_workspace_size(int64_t d, int64_t m, double rho);
rmm_status_t rmm_decode_wq(const void *a, const void *Bq, int32_t fmt, const float *scale, int64_t d, int64_t m,
                           int64_t ldb, double rho, float alpha, void *y, int32_t *idx_out, void *workspace,
                           size_t ws_bytes, hipStream_t stream);

/*
 * The reduced product over 8-bit weights for any number of rows (weight-only
 * quantization, W8A16): RMM on an activation block A and weights stored as
 * 8-bit codes with one fp32 scale per output column, the combination App.
 * B.6 evaluates on INT8-quantized Llama models and App. B.7 leaves to fused
 * quantized kernels.
 *   I = TopK(||A[:, j]||_2, k = rmm_k(rho, d))   (Sec. 3.2: from A alone)
 *   Y[i, c] = alpha * scale[c] * sum_{t<k} A[i, I_t] * q[I_t, c]
 * A: n x d bf16 row-major, leading dimension lda.  Bq: d x m codes, rows ldb
 * bytes apart, fmt RMM_WQ_FP8_E4M3 or RMM_WQ_INT8 (as for rmm_decode_wq).
 * scale: m fp32.  Y: n x m bf16, leading dimension ldy.  idx_out (k int32,
 * ascending) may be NULL.  Every code is exact in bf16, so the kept rows are
 * widened to bf16 inside the kernel and contracted on bf16 MFMA with fp32
 * accumulation; scale[c] and alpha multiply the fp32 sum once and Y is
 * rounded to nearest-even (bit-reproducible: fixed summation order).
 * n = 1 runs rmm_decode_wq (the same result definition, |a_j| scores).
 * Supported for n > 1: n, d, lda, ldy multiples of 8; m and ldb multiples
 * of 16; d < 65535; A, Bq, Y and scale 16-byte aligned; A (and its
 * transpose) and Bq under 2^31 bytes; otherwise RMM_ERR_UNSUPPORTED (the
 * size query returns SIZE_MAX).  workspace: rmm_matmul_wq_workspace_size
 * bytes, 256-byte aligned.  Errors otherwise as for rmm_decode_wq.
 */
size_t rmm_matmul_wq_workspace_size(int64_t n, int64_t d, int64_t m, double rho);
rmm_status_t rmm_matmul_wq(const void *A, int64_t n, int64_t d, int64_t lda, const void *Bq, int32_t fmt,
                           const float *scale, int64_t m, int64_t ldb, double rho, float alpha, void *Y, int64_t ldy,
                           int32_t *idx_out, void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Optional per-kernel timing for measurement tools.  While enabled, every
 * kernel rmm_matmul enqueues is bracketed by a pair of HIP events recorded
 * on the call's stream (at most `capacity` pairs are kept; later kernels are
 * not timed).  rmm_timing_collect synchronizes those events and returns, for
 * each kernel kind k (RMM_KERNEL_*), the summed milliseconds in ms[k] and
 * the launch count in count[k] (arrays of RMM_KERNEL_KINDS entries), then
 * clears the record.  Not thread-safe; meant for a single benchmarking
 * thread.  Enabling allocates the events (host call, outside any capture).
 */
enum {
    RMM_KERNEL_COLNORM = 0,
    RMM_KERNEL_FINALIZE = 1,
    RMM_KERNEL_SELECT = 2,
    RMM_KERNEL_PACK = 3,
    RMM_KERNEL_GEMM = 4,
    RMM_KERNEL_REDUCE = 5,
    RMM_KERNEL_GEMV = 6,
    RMM_KERNEL_OTHER = 7,
    RMM_KERNEL_KINDS = 8
};
rmm_status_t rmm_timing_enable(int32_t enable, int32_t capacity);
rmm_status_t rmm_timing_collect(double *ms, int64_t *count);

/*
 * Matrix-core ceiling probe for measurement tools: enqueues one kernel of
 * `workgroups` workgroups of four waves; each wave issues `iters` rounds of
 * eight independent v_mfma_f32_32x32x16_bf16 (no memory traffic), so the
 * launch performs workgroups * 4 * iters * 8 * 32768 flops.  Timing it
 * (events around the launch) gives the bf16 matrix throughput the chip
 * sustains at the clock it holds under that load, to set beside the
 * datasheet peak.  out: device, out_len >= workgroups * 256 floats (one
 * checksum per thread, written so the work cannot be elided).  clk: device,
 * 2 * workgroups uint64 or NULL; when given, entry 2w receives the shader
 * clock cycles and entry 2w + 1 the ticks of the constant 100 MHz counter
 * that the first wave of workgroup w spent in its loop (clock under this
 * load = cycles / ticks * 100 MHz).
 * Errors: RMM_ERR_INVALID_ARG for NULL out, workgroups outside [1, 2^20],
 * iters < 1 or a short out; RMM_ERR_HIP when the launch fails.
 */
rmm_status_t rmm_calibrate_mfma(int64_t workgroups, int32_t iters, float *out, int64_t out_len, uint64_t *clk,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RMM_H */
