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

// ---------------------------------------------------------------- one-launch decode
// The single-row step's selection and product in one launch: every
// workgroup selects the kept rows itself (the selection depends only on the
// d values of a, 16-32 KB that every workgroup reads from the caches), then
// streams its own block of columns over its split of the kept rows, so no
// workgroup waits for another.  With one split the workgroup writes y; with
// several (about one workgroup per CU in all) it writes fp32 partial sums,
// which one reduce launch adds in split order.
//
// Selection: the key of index j is the magnitude of a_j's bf16 pattern
// (bits 14..0), which orders like |a_j| (NaN above +Inf, -0 = +0).  A
// 256-bin histogram of the top 8 key bits and a 128-bin histogram of the
// low 7 bits inside the bin that holds the k-th largest give the exact
// threshold T and the count of keys above it; every key above T is kept,
// and of the keys equal to T the lowest-indexed ones up to k.  One block
// scan of (above, equal) counts in index order places each kept index at
// its ascending position: the LDS list (row, a value) is ascending, the
// same set and order as the selection kernels produce.
//
// Stream: LPR lanes cover a 16-byte piece each of one kept row's column
// block, so a wave reads 64 / LPR rows per instruction with U instructions
// in flight (as launched, LPR = 64: one 1 KB piece of one row, 512 bf16 or
// 1024 8-bit columns); every lane accumulates its EPL columns over its rows
// in a fixed order, and the workgroup's (1024 / 64) * (64 / LPR) row groups
// are added in a fixed order at the end:
// bit-reproducible.  BQ: 0 = bf16 B, 1 = OCP FP8 E4M3 codes, 2 = int8 codes
// (8-bit: y[c] also times scale[c]).
constexpr int kFusedThreads = 1024;
constexpr int kFusedMaxKeys = 16384;  // d limit (keys per thread <= 16)

template <int BQ, int LPR_>
struct FusedShape {
    static constexpr int EPL = BQ ? 16 : 8;   // columns per lane (one 16-byte load)
    static constexpr int LPR = LPR_;          // lanes per row piece (16-byte pieces)
    static constexpr int CB = EPL * LPR;      // columns per workgroup
    static constexpr int RPI = 64 / LPR;      // rows per wave instruction
};
constexpr int kFusedLpr = 64;  // one 1 KB row piece per wave instruction

__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

template <int BQ, int LPR>
__global__ __launch_bounds__(1024) void decode_fused_kernel(const uint16_t *__restrict__ a, int d, int k,
                                                            const char *__restrict__ B, int64_t row_bytes, int64_t m,
                                                            const float *__restrict__ scale, float alpha,
                                                            uint16_t *__restrict__ y, int32_t *__restrict__ idx_out,
                                                            int rows_per_split, float *__restrict__ part) {
    using S = FusedShape<BQ, LPR>;
    constexpr int E = kFusedMaxKeys / kFusedThreads;
    __shared__ int hist[256];
    __shared__ int wsum[kFusedThreads / 64 + 1];
    __shared__ int sinfo[4];
    __shared__ uint16_t sidx[kFusedMaxKeys];
    __shared__ float sval[kFusedMaxKeys];  // then the row-group sums (row groups x CB floats)
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    // ---- keys: `per` consecutive indices per thread
    const int per = (d + kFusedThreads - 1) / kFusedThreads;
    const int j0 = tid * per;
    uint32_t raw[E];
#pragma unroll
    for (int e = 0; e < E; ++e) raw[e] = (e < per && j0 + e < d) ? (uint32_t)a[j0 + e] : 0x10000u;  // 0x10000: no key
    for (int q = tid; q < 256; q += kFusedThreads) hist[q] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (raw[e] < 0x10000u) atomicAdd(&hist[(raw[e] & 0x7fffu) >> 7], 1);
    __syncthreads();
    if (w == 0) {
        // bins in descending order, four per lane: the bin holding the k-th largest key
        int c[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c[q] = hist[255 - 4 * lane - q];
            sum += c[q];
        }
        const int incl = wave_incl_scan_i32(sum, lane);
        int above = incl - sum;
        if (above < k && k <= incl) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (above + c[q] >= k) {
                    sinfo[0] = 255 - 4 * lane - q;
                    sinfo[1] = above;
                    break;
                }
                above += c[q];
            }
        }
    }
    __syncthreads();
    const uint32_t b1 = (uint32_t)sinfo[0];
    for (int q = tid; q < 128; q += kFusedThreads) hist[q] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (raw[e] < 0x10000u && ((raw[e] & 0x7fffu) >> 7) == b1) atomicAdd(&hist[raw[e] & 0x7fu], 1);
    __syncthreads();
    if (w == 0) {
        const int above1 = sinfo[1];
        int c[2], sum = 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            c[q] = hist[127 - 2 * lane - q];
            sum += c[q];
        }
        const int incl = above1 + wave_incl_scan_i32(sum, lane);
        int above = incl - sum;
        if (above < k && k <= incl) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (above + c[q] >= k) {
                    sinfo[2] = (int)((b1 << 7) | (uint32_t)(127 - 2 * lane - q));
                    sinfo[3] = above;
                    break;
                }
                above += c[q];
            }
        }
    }
    __syncthreads();
    const uint32_t T = (uint32_t)sinfo[2];
    const int need_eq = k - sinfo[3];
    // ---- ascending compaction: block scan of (keys above T) << 16 | (keys equal to T)
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (raw[e] >= 0x10000u) continue;
        const uint32_t kk = raw[e] & 0x7fffu;
        gt += kk > T;
        eq += kk == T;
    }
    const int v = (gt << 16) | eq;
    const int incl = wave_incl_scan_i32(v, lane);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
        const int t = lane < kFusedThreads / 64 ? wsum[lane] : 0;
        const int u = wave_incl_scan_i32(t, lane);
        if (lane < kFusedThreads / 64) wsum[lane] = u - t;
    }
    __syncthreads();
    const int excl = wsum[w] + incl - v;
    int gb = excl >> 16, eb = excl & 0xffff;
    const bool write_idx = idx_out && blockIdx.x == 0 && blockIdx.y == 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (raw[e] >= 0x10000u) continue;
        const uint32_t kk = raw[e] & 0x7fffu;
        int t = -1;
        if (kk > T) {
            t = gb + min(eb, need_eq);
            ++gb;
        } else if (kk == T) {
            if (eb < need_eq) t = gb + eb;
            ++eb;
        }
        if (t >= 0) {
            sidx[t] = (uint16_t)(j0 + e);
            sval[t] = __uint_as_float(raw[e] << 16);
            if (write_idx) idx_out[t] = j0 + e;
        }
    }
    __syncthreads();

    // ---- stream the workgroup's column block over every kept row
    const int g = lane / S::LPR, cl = lane % S::LPR;
    const int64_t c0 = (int64_t)blockIdx.x * S::CB + cl * S::EPL;
    const bool col_ok = c0 < m;
    const char *Bc = B + c0 * (BQ ? 1 : 2);
    float acc[S::EPL];
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) acc[e] = 0.f;
    constexpr int U = 8;                                   // loads in flight per lane
    constexpr int ROUND = (kFusedThreads / 64) * S::RPI;  // rows per wave-round of the workgroup
    const int t_lo = (int)blockIdx.y * rows_per_split, t_hi = min(k, t_lo + rows_per_split);
    for (int tb = t_lo; tb < t_hi; tb += ROUND * U) {
        uint4 vv[U];
        float av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tb + u * ROUND + w * S::RPI + g;
            const bool ok = t < t_hi && col_ok;
            av[u] = ok ? sval[t] : 0.f;
            vv[u] = ok ? *reinterpret_cast<const uint4 *>(Bc + (int64_t)sidx[t] * row_bytes) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (BQ == 0) {
                fma8(acc, av[u], vv[u]);
            } else {
                fma4_q8<BQ - 1>(acc, av[u], vv[u].x);
                fma4_q8<BQ - 1>(acc + 4, av[u], vv[u].y);
                fma4_q8<BQ - 1>(acc + 8, av[u], vv[u].z);
                fma4_q8<BQ - 1>(acc + 12, av[u], vv[u].w);
            }
        }
    }
    __syncthreads();  // every wave is done with the list: its LDS takes the row-group sums
    float *red = sval;
    const int rg = w * S::RPI + g;
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) red[rg * S::CB + cl * S::EPL + e] = acc[e];
    __syncthreads();
    constexpr int NRG = (kFusedThreads / 64) * S::RPI;  // row groups
    static_assert(NRG * S::CB <= kFusedMaxKeys, "row-group sums fit in the list's LDS");
    for (int c = tid; c < S::CB; c += kFusedThreads) {
        const int64_t col = (int64_t)blockIdx.x * S::CB + c;
        float sum = 0.f;
        for (int r = 0; r < NRG; ++r) sum += red[r * S::CB + c];
        if (col < m) {
            if (part) {  // split rows: scaled partial sums, alpha applied by the reduce
                part[(int64_t)blockIdx.y * m + col] = BQ ? sum * scale[col] : sum;
            } else {
                const float f = BQ ? alpha * scale[col] : alpha;
                y[col] = f32_to_bf16(f * sum);
            }
        }
    }
}

}  // namespace

int64_t decode_fused_min_m() { return 28 * FusedShape<0, kFusedLpr>::CB; }

int decode_fused_splits(int bq, int64_t m, int64_t k) {
    // about one workgroup per CU (each selects once), whole column blocks
    const int64_t cb = bq ? FusedShape<1, kFusedLpr>::CB : FusedShape<0, kFusedLpr>::CB;
    const int64_t blocks = (m + cb - 1) / cb;
    int64_t s = 256 / blocks;
    const int64_t max_s = (k + 255) / 256;  // at least 256 kept rows per split
    if (s > max_s) s = max_s;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_decode_fused(const uint16_t *a, int64_t d, int64_t k, const void *B, int bq, int64_t ldb, int64_t m,
                               const float *scale, float alpha, uint16_t *y, int32_t *idx_out, int splits,
                               float *part, hipStream_t stream) {
    if (d < 1 || d > kFusedMaxKeys || k < 1 || k > d || m < 1 || bq < 0 || bq > 2 || (bq && !scale) ||
        m % (bq ? 16 : 8) || ldb % (bq ? 16 : 8) || splits < 1 || (splits > 1 && !part))
        return hipErrorInvalidValue;
    const int64_t cb = bq ? FusedShape<1, kFusedLpr>::CB : FusedShape<0, kFusedLpr>::CB;
    const dim3 grid((unsigned)((m + cb - 1) / cb), (unsigned)splits);
    const int rps = (int)((k + splits - 1) / splits);
    float *pp = splits > 1 ? part : nullptr;
    const char *Bb = static_cast<const char *>(B);
    if (bq == 0)
        decode_fused_kernel<0, kFusedLpr><<<grid, kFusedThreads, 0, stream>>>(a, (int)d, (int)k, Bb, ldb * 2, m, scale,
                                                                              alpha, y, idx_out, rps, pp);
    else if (bq == 1)
        decode_fused_kernel<1, kFusedLpr><<<grid, kFusedThreads, 0, stream>>>(a, (int)d, (int)k, Bb, ldb, m, scale,
                                                                              alpha, y, idx_out, rps, pp);
    else
        decode_fused_kernel<2, kFusedLpr><<<grid, kFusedThreads, 0, stream>>>(a, (int)d, (int)k, Bb, ldb, m, scale,
                                                                              alpha, y, idx_out, rps, pp);
    return hipGetLastError();
}

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
