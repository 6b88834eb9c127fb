// Gathered GEMV for single-row decode on gfx950.
//
// With one activation row (n = 1) the score of index j is just |a_j| and the
// reduced product y = sum_{t<k} a[I_t] B[I_t, :] reads k of B's d rows once
// ("Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction for
// LLM Inference", App. D.1: per-step decode cost falls from O(tD) to
// O(rho t D)).  At one multiply-add per two bytes of B this is HBM-bound, so
// the kernel is built for streaming: a workgroup owns 512 columns and one
// split of the kept rows; it first copies that split's row numbers and
// activation values a[I_t] into LDS, then each of its 8 waves reads 1 KB of
// one kept row per instruction (16 bytes per lane) with 8 rows in flight,
// the waves taking interleaved rows.  Partial sums are combined across waves
// in LDS and across splits by splitk_reduce, both in a fixed order (no
// atomics, bit-reproducible).
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kGemvCols = 512;     // columns per workgroup (64 lanes x 8)
constexpr int kGemvWaves = 8;
constexpr int kGemvMaxRows = 2048;  // kept rows per split (LDS copy of the list)

__device__ __forceinline__ void fma8(float (&acc)[8], float a, uint4 v) {
    acc[0] = fmaf(a, __uint_as_float(v.x << 16), acc[0]);
    acc[1] = fmaf(a, __uint_as_float(v.x & 0xffff0000u), acc[1]);
    acc[2] = fmaf(a, __uint_as_float(v.y << 16), acc[2]);
    acc[3] = fmaf(a, __uint_as_float(v.y & 0xffff0000u), acc[3]);
    acc[4] = fmaf(a, __uint_as_float(v.z << 16), acc[4]);
    acc[5] = fmaf(a, __uint_as_float(v.z & 0xffff0000u), acc[5]);
    acc[6] = fmaf(a, __uint_as_float(v.w << 16), acc[6]);
    acc[7] = fmaf(a, __uint_as_float(v.w & 0xffff0000u), acc[7]);
}

// grid: (ceil(m / 512), splits); block 512.  part[split][m].
__global__ __launch_bounds__(512) void gemv_partial_kernel(const uint16_t *__restrict__ B, int64_t ldb, int64_t m,
                                                           const int32_t *__restrict__ idx,
                                                           const float *__restrict__ aval, int64_t k,
                                                           int64_t rows_per_split, float *__restrict__ part) {
    __shared__ float red[kGemvWaves][kGemvCols];
    __shared__ int32_t srow[kGemvMaxRows];
    __shared__ float sval[kGemvMaxRows];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * kGemvCols + lane * 8;
    const int64_t t0 = (int64_t)blockIdx.y * rows_per_split;
    const int nt = (int)max((int64_t)0, min(k, t0 + rows_per_split) - t0);
    for (int q = threadIdx.x; q < nt; q += 512) {
        srow[q] = idx[t0 + q];
        sval[q] = aval[t0 + q];
    }
    __syncthreads();
    const bool col_ok = c0 < m;  // m % 8 == 0 on this path
    const uint16_t *Bc = B + c0;

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    int t = wave;
    if (col_ok) {
        constexpr int U = 8;  // rows in flight per wave
        for (; t + (U - 1) * kGemvWaves < nt; t += U * kGemvWaves) {
            uint4 v[U];
            float a[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t g = srow[t + u * kGemvWaves];
                a[u] = sval[t + u * kGemvWaves];
                v[u] = *reinterpret_cast<const uint4 *>(Bc + g * ldb);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) fma8(acc, a[u], v[u]);
        }
        for (; t < nt; t += kGemvWaves) {
            const int64_t g = srow[t];
            fma8(acc, sval[t], *reinterpret_cast<const uint4 *>(Bc + g * ldb));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
    __syncthreads();
    for (int c = threadIdx.x; c < kGemvCols; c += 512) {
        const int64_t col = (int64_t)blockIdx.x * kGemvCols + c;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kGemvWaves; ++w) sum += red[w][c];
        if (col < m) part[(int64_t)blockIdx.y * m + col] = sum;
    }
}

// The same gathered GEMV over weights stored in 8 bits with one fp32 scale
// per output column (weight-only quantization, W8A16): B holds codes q,
// B[t, c] = q[t, c] * scale[c], so y_c = scale[c] * sum_t a[I_t] q[I_t, c].
// Half the bytes of bf16 weights for the same rows.  FMT 0: OCP FP8 E4M3
// codes, decoded by the gfx950 conversion instruction; FMT 1: int8.  A wave
// reads 1 KB (1024 columns) of one kept row per instruction; each lane keeps
// sixteen fp32 sums and the scale is applied once, to the workgroup's sum.
constexpr int kGemvWqCols = 1024;

template <int FMT>
__device__ __forceinline__ void fma4_q8(float *acc, float a, uint32_t w) {
    if constexpr (FMT == 0) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
        acc[0] = fmaf(a, lo[0], acc[0]);
        acc[1] = fmaf(a, lo[1], acc[1]);
        acc[2] = fmaf(a, hi[0], acc[2]);
        acc[3] = fmaf(a, hi[1], acc[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(a, (float)((int32_t)(w << (24 - 8 * i)) >> 24), acc[i]);
    }
}

// grid: (ceil(m / 1024), splits); block 512.  part[split][m].
template <int FMT>
__global__ __launch_bounds__(512) void gemv_wq_partial_kernel(const uint8_t *__restrict__ B, int64_t ldb, int64_t m,
                                                              const float *__restrict__ scale,
                                                              const int32_t *__restrict__ idx,
                                                              const float *__restrict__ aval, int64_t k,
                                                              int64_t rows_per_split, float *__restrict__ part) {
    __shared__ float red[kGemvWaves][kGemvWqCols];
    __shared__ int32_t srow[kGemvMaxRows];
    __shared__ float sval[kGemvMaxRows];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * kGemvWqCols + lane * 16;
    const int64_t t0 = (int64_t)blockIdx.y * rows_per_split;
    const int nt = (int)max((int64_t)0, min(k, t0 + rows_per_split) - t0);
    for (int q = threadIdx.x; q < nt; q += 512) {
        srow[q] = idx[t0 + q];
        sval[q] = aval[t0 + q];
    }
    __syncthreads();
    const bool col_ok = c0 < m;  // m % 16 == 0 on this path
    const uint8_t *Bc = B + c0;

    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;

    int t = wave;
    if (col_ok) {
        constexpr int U = 8;  // rows in flight per wave
        for (; t + (U - 1) * kGemvWaves < nt; t += U * kGemvWaves) {
            uint4 v[U];
            float a[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t g = srow[t + u * kGemvWaves];
                a[u] = sval[t + u * kGemvWaves];
                v[u] = *reinterpret_cast<const uint4 *>(Bc + g * ldb);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                fma4_q8<FMT>(acc, a[u], v[u].x);
                fma4_q8<FMT>(acc + 4, a[u], v[u].y);
                fma4_q8<FMT>(acc + 8, a[u], v[u].z);
                fma4_q8<FMT>(acc + 12, a[u], v[u].w);
            }
        }
        for (; t < nt; t += kGemvWaves) {
            const int64_t g = srow[t];
            const uint4 v = *reinterpret_cast<const uint4 *>(Bc + g * ldb);
            fma4_q8<FMT>(acc, sval[t], v.x);
            fma4_q8<FMT>(acc + 4, sval[t], v.y);
            fma4_q8<FMT>(acc + 8, sval[t], v.z);
            fma4_q8<FMT>(acc + 12, sval[t], v.w);
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][lane * 16 + e] = acc[e];
    __syncthreads();
    for (int c = threadIdx.x; c < kGemvWqCols; c += 512) {
        const int64_t col = (int64_t)blockIdx.x * kGemvWqCols + c;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kGemvWaves; ++w) sum += red[w][c];
        if (col < m) part[(int64_t)blockIdx.y * m + col] = sum * scale[col];
    }
}

}  // namespace

int gemv_wq_splits(int64_t m, int64_t k) {
    // about 1024 workgroups of 1024 columns, at least 256 kept rows per split
    // (an 8-bit row is half a bf16 row: longer splits amortise each
    // workgroup's list copy and LDS sum)
    const int64_t blocks = (m + kGemvWqCols - 1) / kGemvWqCols;
    int64_t s = (1024 + blocks - 1) / blocks;
    const int64_t max_s = (k + 255) / 256;
    if (s > max_s) s = max_s;
    const int64_t min_s = (k + kGemvMaxRows - 1) / kGemvMaxRows;
    if (s < min_s) s = min_s;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_gemv_wq_partial(const uint8_t *B, int fmt, int64_t ldb, int64_t m, const float *scale,
                                  const int32_t *idx, const float *aval, int64_t k, int splits, float *part,
                                  hipStream_t stream) {
    const int64_t rows_per_split = (k + splits - 1) / splits;
    if (rows_per_split > kGemvMaxRows || m % 16 || ldb % 16 || (fmt != 0 && fmt != 1)) return hipErrorInvalidValue;
    dim3 grid((unsigned)((m + kGemvWqCols - 1) / kGemvWqCols), (unsigned)splits);
    if (fmt == 0)
        gemv_wq_partial_kernel<0><<<grid, 512, 0, stream>>>(B, ldb, m, scale, idx, aval, k, rows_per_split, part);
    else
        gemv_wq_partial_kernel<1><<<grid, 512, 0, stream>>>(B, ldb, m, scale, idx, aval, k, rows_per_split, part);
    return hipGetLastError();
}

int gemv_splits(int64_t m, int64_t k) {
    // about 2048 workgroups (eight per CU: enough rows in flight to keep HBM
    // busy), at least 128 kept rows per split and at most kGemvMaxRows
    const int64_t blocks = (m + kGemvCols - 1) / kGemvCols;
    int64_t s = (2048 + blocks - 1) / blocks;
    const int64_t max_s = (k + 127) / 128;
    if (s > max_s) s = max_s;
    const int64_t min_s = (k + kGemvMaxRows - 1) / kGemvMaxRows;
    if (s < min_s) s = min_s;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_gemv_partial(const uint16_t *B, int64_t ldb, int64_t m, const int32_t *idx, const float *aval,
                               int64_t k, int splits, float *part, hipStream_t stream) {
    const int64_t rows_per_split = (k + splits - 1) / splits;
    if (rows_per_split > kGemvMaxRows) return hipErrorInvalidValue;
    dim3 grid((unsigned)((m + kGemvCols - 1) / kGemvCols), (unsigned)splits);
    gemv_partial_kernel<<<grid, 512, 0, stream>>>(B, ldb, m, idx, aval, k, rows_per_split, part);
    return hipGetLastError();
}

}  // namespace rmm
