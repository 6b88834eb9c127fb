// Gathered GEMV for single-row decode on gfx950.
//
// With one activation row (n = 1) the score of index j is just |a_j| and the
// reduced product y = sum_{t<k} a[I_t] B[I_t, :] reads k of B's d rows once
// ("Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction for
// LLM Inference", App. D.1: per-step decode cost falls from O(tD) to
// O(rho t D)).  At one multiply-add per two bytes of B this is HBM-bound, so
// the kernel is built for streaming: each wave reads 1 KB of one kept row per
// instruction (16 bytes per lane), four rows are in flight per wave, the four
// waves of a workgroup take interleaved rows of one K split, and partial sums
// are combined first across waves in LDS and then across splits, both in a
// fixed order (no atomics, bit-reproducible).  The kept row numbers and
// activation values a[I_t] are wave-uniform and come from the selection
// kernel's outputs.
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kGemvCols = 512;  // columns per workgroup (64 lanes x 8)

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

// grid: (ceil(m / 512), splits); block 256.  part[split][m].
__global__ __launch_bounds__(256) void gemv_partial_kernel(const uint16_t *__restrict__ B, int64_t ldb, int64_t m,
                                                           const int32_t *__restrict__ idx,
                                                           const float *__restrict__ aval, int64_t k,
                                                           int64_t rows_per_split, float *__restrict__ part) {
    __shared__ float red[4][kGemvCols];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * kGemvCols + lane * 8;
    const int64_t t0 = (int64_t)blockIdx.y * rows_per_split;
    const int64_t t1 = min(k, t0 + rows_per_split);
    const bool col_ok = c0 < m;  // m % 8 == 0 on this path
    const uint16_t *Bc = B + c0;

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    int64_t t = t0 + wave;
    if (col_ok) {
        for (; t + 12 < t1; t += 16) {
            const int64_t g0 = idx[t], g1 = idx[t + 4], g2 = idx[t + 8], g3 = idx[t + 12];
            const float a0 = aval[t], a1 = aval[t + 4], a2 = aval[t + 8], a3 = aval[t + 12];
            const uint4 v0 = *reinterpret_cast<const uint4 *>(Bc + g0 * ldb);
            const uint4 v1 = *reinterpret_cast<const uint4 *>(Bc + g1 * ldb);
            const uint4 v2 = *reinterpret_cast<const uint4 *>(Bc + g2 * ldb);
            const uint4 v3 = *reinterpret_cast<const uint4 *>(Bc + g3 * ldb);
            fma8(acc, a0, v0);
            fma8(acc, a1, v1);
            fma8(acc, a2, v2);
            fma8(acc, a3, v3);
        }
        for (; t < t1; t += 4) {
            const int64_t g0 = idx[t];
            const uint4 v0 = *reinterpret_cast<const uint4 *>(Bc + g0 * ldb);
            fma8(acc, aval[t], v0);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
    __syncthreads();
    for (int c = threadIdx.x; c < kGemvCols; c += 256) {
        const int64_t col = (int64_t)blockIdx.x * kGemvCols + c;
        if (col < m) part[(int64_t)blockIdx.y * m + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    }
}

}  // namespace

int gemv_splits(int64_t m, int64_t k) {
    const int64_t blocks = (m + kGemvCols - 1) / kGemvCols;
    int64_t s = (1024 + blocks - 1) / blocks;
    const int64_t max_s = (k + 63) / 64;  // at least 64 rows (16 per wave) per split
    if (s > max_s) s = max_s;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_gemv_partial(const uint16_t *B, int64_t ldb, int64_t m, const int32_t *idx, const float *aval,
                               int64_t k, int splits, float *part, hipStream_t stream) {
    const int64_t rows_per_split = (k + splits - 1) / splits;
    dim3 grid((unsigned)((m + kGemvCols - 1) / kGemvCols), (unsigned)splits);
    gemv_partial_kernel<<<grid, 256, 0, stream>>>(B, ldb, m, idx, aval, k, rows_per_split, part);
    return hipGetLastError();
}

}  // namespace rmm
