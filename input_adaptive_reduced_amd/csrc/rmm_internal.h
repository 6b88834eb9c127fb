// Internal declarations shared by the HIP translation units of librmm.
// Not installed; the public interface is include/rmm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmm.h"

namespace rmm {

// ---------------------------------------------------------------- bf16 helpers (device)
// bf16 is carried as its raw 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Two floats rounded to bf16 (nearest-even) and packed low/high into one
// word with the hardware conversion: one v_cvt_pk_bf16_f32, bit-identical
// to f32_to_bf16 for every finite input (NaN stays NaN).
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 rmm_bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float rmm_f32x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const rmm_f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, rmm_bf16x2_t));
}

// Order-preserving map from an fp32 score to an unsigned key (larger score ->
// larger key).  -0 is folded onto +0 and every NaN onto +qNaN, which ranks
// above +Inf.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) u = 0x7fc00000u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- kernel kinds (timing)
struct Timer;  // host-side per-launch event recorder (rmm_api.hip)
void timing_begin(hipStream_t s, int kind);
void timing_end(hipStream_t s, int kind);

// ---------------------------------------------------------------- launchers (host)
// All launchers enqueue on `stream` and return hipGetLastError().

// Partial sums of squares per column: part[b][r][j] = sum over rows of chunk r.
// Grid shape is chosen by colnorm_plan().
struct ColnormPlan {
    int tc;          // threads per row (columns / vec)
    int strips;      // column strips
    int chunks;      // row chunks R
    int64_t rows_per_chunk;
    int rpt;         // bf16: rows per thread with every load issued up front (0: looped kernel)
};
ColnormPlan colnorm_plan(rmm_dtype_t dt, int64_t n, int64_t d, int64_t batch);
hipError_t launch_colnorm_partial(const void *A, rmm_dtype_t dt, int64_t n, int64_t d, int64_t lda,
                                  int64_t batch, int64_t strideA, const ColnormPlan &p, float *part,
                                  hipStream_t stream);
// The same partials (one batch entry, bf16) from a pass that also writes
// At = A^T (d x n, rows ldt apart), the gather source of gemm_tdma_kernel.
// n, d, lda and ldt multiples of 8; A and At 16-byte aligned.  The plan's
// rpt field holds the 128-row tiles per row chunk (1, 2 or 4).
ColnormPlan colnorm_transpose_plan(int64_t n, int64_t d);
hipError_t launch_colnorm_transpose(const void *A, int64_t n, int64_t d, int64_t lda, const ColnormPlan &p,
                                    uint16_t *At, int64_t ldt, float *part, hipStream_t stream);
// s[b][j] = sqrt(sum_r part[b][r][j]) in a fixed order.
hipError_t launch_colnorm_finalize(const float *part, int64_t chunks, int64_t d, int64_t batch, float *s,
                                   hipStream_t stream);
// Longest score vector the register-resident selection (select_kernel,
// norm_select_kernel, the decode |a| selection) handles; longer ones use
// select_big_kernel.
constexpr int64_t kFusedSelectMaxD = 16384;
// Norms from the row-chunk partials and the selection in one launch (one
// workgroup per batch entry, every partial load in flight at once).  One
// workgroup reads all chunks x d partials, so this pays only while they are
// few: d <= 16384 and at most 256 KB of partials (beyond that, on MI355X, a
// wide finalize launch plus the selection launch is faster: 459 KB at
// d = 14336 took 18.8 us against 3.7 + 12.0).  d % 4 == 0, part 16-byte
// aligned.
inline bool norm_select_ok(int64_t chunks, int64_t d) {
    return d % 4 == 0 && d <= 16384 && chunks * d <= 65536;
}
hipError_t launch_norm_select(const float *part, int64_t chunks, int64_t d, int64_t batch, int64_t k, int32_t *idx,
                              int64_t ld_idx, int32_t *idx_pad, int64_t ld_pad, hipStream_t stream);

// Exact TopK by radix select; rows of idx (ld_idx apart) and of idx_pad
// (ld_pad apart, entries k..ld_pad-1 set to -1) receive the kept indices in
// ascending order; either may be null.  When `a_src` is given the scores are
// |a_j| of a single bf16/f32 row per batch entry (decode) and `aval[b*k + t]`
// receives a[idx[t]] as fp32.
hipError_t launch_select(const float *s, const void *a_src, rmm_dtype_t a_dt, int64_t a_stride, int64_t batch,
                         int64_t d, int64_t k, int32_t *idx, int64_t ld_idx, int32_t *idx_pad, int64_t ld_pad,
                         float *aval, hipStream_t stream);

// dst[b][r][t] = src[b / group][r][idx[b][t]] for t < kpad, 0 where idx[b][t]
// is -1.  idx rows are ld_idx apart (a multiple of 64, 256-byte aligned).
// layout 0: dst rows of kpad entries (row r at dst + r * kpad).
// layout 1: MFMA operand blocks for the A-direct GEMM: rows padded to a
// multiple of 32; the 16-byte piece (row r, entries 8c..8c+7) sits at element
// ((r / 32) * (kpad / 16) + c / 2) * 512 + ((c % 2) * 32 + r % 32) * 8.
hipError_t launch_pack(const void *src, rmm_dtype_t dt, int64_t rows, int64_t d, int64_t ld_src,
                       int64_t src_stride, int64_t group, const int32_t *idx, int64_t ld_idx, int64_t kpad,
                       void *dst, int64_t dst_stride, int64_t batch, int layout, hipStream_t stream);

// Selection and layout-1 pack in one launch for short rows (d = 64 or 128,
// attention head dimensions): per batch entry b, the kept set of the column
// norms whose row-chunk partials are part[b][chunk][0..d) (the same sums,
// keys and tie order as launch_norm_select), written to idx[b * ld_idx ..]
// (k entries, when idx is given) and pad[b * kpad ..] (kpad entries, -1 past
// k), and dst[b] = src[b / group][:, kept] as launch_pack with layout 1.
// Needs k <= kpad <= d, kpad % 64 == 0, at most kSelectPackMaxChunks chunks,
// 16-byte aligned src rows and dst.
constexpr int64_t kSelectPackMaxChunks = 64;
bool select_pack_short_ok(int64_t d, int64_t k, int64_t kpad, int64_t chunks);
hipError_t launch_select_pack_short(const float *part, int64_t chunks, int64_t k, int32_t *idx, int64_t ld_idx,
                                    int32_t *pad, int64_t kpad, const void *src, int64_t rows, int64_t d,
                                    int64_t ld_src, int64_t src_stride, int64_t group, void *dst, int64_t dst_stride,
                                    int64_t batch, hipStream_t stream);

// A caller-supplied index set (batch rows of k int32, row b at idx + b*k)
// into the padded list: entries in [0, d) that exceed every earlier in-range
// entry of their row, compacted ascending, then -1 up to ld_pad.  With a_row
// (a bf16 decode row, batch 1) the kept values go to aval[0..k) and the
// slots after the kept ones up to k hold row 0 with value 0.
hipError_t launch_index_prepare(const int32_t *idx, int64_t batch, int64_t k, int64_t d, int32_t *idx_pad,
                                int64_t ld_pad, const void *a_row, float *aval, hipStream_t stream);

// Index rows 0..k-1 then -1 up to ld, per batch entry (rho = 1 shortcut).
hipError_t launch_iota(int32_t *idx, int64_t k, int64_t ld, int64_t batch, hipStream_t stream);

// bf16 MFMA GEMM  Y = alpha * Ap[:, 0:k] * Bsel  (see gemm.hip for operand modes).
struct GemmArgs {
    const uint16_t *A;   // packed/dense A, k-contiguous rows
    int64_t lda, strideA;
    const uint16_t *B;   // bmode 0: d x m row-major rows gathered by idx; bmode 1: m x k k-contiguous
    int64_t ldb, strideB;
    int64_t group;       // batch entries sharing one B (B + (b / group) * strideB)
    const int32_t *idx;  // bmode 0: padded row list per entry (-1 beyond k), ld_idx apart
    int64_t ld_idx;
    uint16_t *Y;
    int64_t ldy, strideY;
    float *part;         // split-K fp32 partials [split][batch][n][m] (NULL = no split)
    int64_t n, m, k, kpad, batch;
    int64_t a_bytes;     // bytes readable from each entry's A base (< 2^31)
    int64_t b_bytes;     // bytes readable from each B base (< 2^31)
    int splits;
    int bmode;
    float alpha;
    int epi;             // tile 5 only: 0 = Y, 1 = SwiGLU of interleaved gate/up column blocks (see gemm.hip)
    uint16_t *Yt;        // epi 1: h^T (m/2 x n, rows n apart), or NULL
    float *npart;        // epi 1 with Yt: column sums of h^2 per 256-row chunk [chunk][m/2]
    int bq;              // tile 5 only: B element format, 0 = bf16, 1 = OCP FP8 E4M3 codes, 2 = int8 codes
                         // (8-bit B: ldb in bytes, rows of m codes; b_bytes in bytes)
    const float *colscale;  // bq != 0: one fp32 scale per output column (Y = alpha * scale[c] * sum)
};
struct GemmConfig {
    int tile;    // 0: 256x256, 1: 128x128, 2: 256x256 with A in operand blocks (A-direct),
                 // 3: persistent single-K-step kernel, both operands in operand blocks,
                 // 4: as 2 with B rows staged by LDS-DMA loads (gemm_bdma_kernel),
                 // 5: both operands gathered by rows into LDS (gemm_tdma_kernel;
                 //    A is then A^T, d x n, lda = its row length),
                 // 6: narrow output, A read in place with its kept columns gathered in
                 //    the kernel (gemm_gcol_kernel; m <= kGcolMaxM, d <= kGcolMaxD, d % 8 == 0)
    int splits;  // >= 1
};
// Largest output width and contraction length of tile 6.
constexpr int64_t kGcolMaxM = 128;
constexpr int64_t kGcolMaxD = 8192;
GemmConfig gemm_choose(int64_t n, int64_t m, int64_t k, int64_t batch, int64_t d, int transB);
// Tile 5 with its K splits for a single product whose A is given transposed,
// or tile -1 when the shape does not suit it.
GemmConfig gemm_choose_transposed(int64_t n, int64_t m, int64_t k, int64_t d);
// Whether tile 5 can run a K range of kpad padded entries in `splits` splits
// (its kept-row list must fit in LDS) for contraction length d; bq != 0: with
// 8-bit B, whose smaller stages leave room for a longer list.
bool gemm_tdma_fits(int64_t kpad, int splits, int64_t d, int bq = 0);
hipError_t launch_gemm_bf16(const GemmArgs &g, const GemmConfig &c, hipStream_t stream);
// Gate and up weights of a gated MLP (d x m each; stored m x d, the nn.Linear
// layout, when `transposed`) interleaved in 32-column blocks into one d x 2m
// operand: columns 64c..64c+31 = gate columns 32c.., 64c+32..64c+63 = up
// columns 32c..  m % 32 == 0, 16-byte aligned output.
hipError_t launch_gated_weights(const uint16_t *Wg, const uint16_t *Wu, int64_t d, int64_t m, int transposed,
                                uint16_t *Wgu, hipStream_t stream);
// Y = alpha * sum_s part[s] (s ascending), rounded to bf16.
hipError_t launch_splitk_reduce(const float *part, int splits, int64_t n, int64_t m, int64_t batch, float alpha,
                                uint16_t *Y, int64_t ldy, int64_t strideY, hipStream_t stream);

// Generic gathered GEMM for any dtype, alignment and shape (SIMT fp32 FMA).
struct GenericArgs {
    rmm_dtype_t dt;
    const void *A;
    int64_t lda, strideA;
    const void *B;
    int64_t ldb, strideB, group;
    int transB;
    const int32_t *idx;  // NULL = identity
    int64_t ld_idx;
    void *Y;
    int64_t ldy, strideY;
    int64_t n, m, k, batch;
    float alpha;
};
hipError_t launch_gemm_generic(const GenericArgs &g, hipStream_t stream);

// Decode: y = alpha * sum_t aval[t] * B[idx[t], :] (split over t, then reduce).
// Attention with reduced scores and the softmax fused (attention.hip).  K
// packed per query head in MFMA operand blocks (launch_pack layout 1, kq = 64
// or 128 entries per row), Q as given, V row-major (Lk x 128 per key/value head,
// ldv apart), O row-major (Lq x 128 per query head, ldo apart).  *_stride
// are per-head element strides, *_bytes the bytes readable from each head's
// base (< 2^31).  scale_log2 = alpha * log2(e).
struct AttnArgs {
    const uint16_t *Q;     // H x Lq x dh row-major (the kept columns are gathered in the kernel)
    const int32_t *idx;    // kept columns per head, ld_idx apart, -1 past k
    int64_t ld_idx, dh;
    const uint16_t *K;
    int64_t k_stride, k_bytes;
    const uint16_t *V;
    int64_t ldv, v_stride, v_bytes;
    uint16_t *O;
    int64_t ldo, o_stride;
    int H, group, Lq, Lk, causal;
    int pair;  // causal query tiles paired per workgroup (set by launch_attention_fwd)
    float scale_log2;
};
hipError_t launch_attention_fwd(const AttnArgs &a, int kq, hipStream_t stream);

int gemv_splits(int64_t m, int64_t k);
// Single-row decode with the selection inside the GEMV: every workgroup
// selects from |a| itself (a bf16, d <= 16384), then streams one 512-column
// (bf16 B, bq 0) or 1024-column (8-bit codes, bq 1 = FP8 E4M3, 2 = int8,
// with per-column scale) block over one split of the kept rows; ldb in
// elements.  splits == 1: y[c] = alpha (* scale[c]) * sum_t a[I_t] B[I_t, c]
// rounded to bf16; otherwise part[split][c] (scaled, without alpha) for
// launch_splitk_reduce.  idx_out (k int32, ascending) may be NULL.  Taken
// for wide outputs (m >= decode_fused_min_m()), with decode_fused_splits
// splits (about one workgroup per CU).
int64_t decode_fused_min_m();
int decode_fused_splits(int bq, int64_t m, int64_t k);
hipError_t launch_decode_fused(const uint16_t *a, int64_t d, int64_t k, const void *B, int bq, int64_t ldb, int64_t m,
                               const float *scale, float alpha, uint16_t *y, int32_t *idx_out, int splits,
                               float *part, hipStream_t stream);
// Gathered GEMV over 8-bit weights (fmt 0: OCP FP8 E4M3, 1: int8) with one
// fp32 scale per column: part[split][c] = scale[c] * sum over the split's
// kept rows of aval[t] * q[idx[t], c].  m and ldb multiples of 16, B 16-byte
// aligned.
int gemv_wq_splits(int64_t m, int64_t k);
hipError_t launch_gemv_wq_partial(const uint8_t *B, int fmt, int64_t ldb, int64_t m, const float *scale,
                                  const int32_t *idx, const float *aval, int64_t k, int splits, float *part,
                                  hipStream_t stream);
hipError_t launch_gemv_partial(const uint16_t *B, int64_t ldb, int64_t m, const int32_t *idx, const float *aval,
                               int64_t k, int splits, float *part, hipStream_t stream);

}  // namespace rmm
