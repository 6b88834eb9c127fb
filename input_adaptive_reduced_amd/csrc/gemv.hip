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

}  // namespace

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
