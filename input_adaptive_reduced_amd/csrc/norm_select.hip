// Column norms and exact TopK selection for gfx950.
//
// Steps 1 and 2 of reduced matrix multiplication ("Reduced Matrix
// Multiplication: Input-Adaptive Matrix-Product Reduction for LLM Inference",
// Sec. 3.2): the score of contraction index j is s_j = ||A[:, j]||_2 over all
// rows of the current activation block, and the kept set is the ceil(rho d)
// largest scores.  Sec. 3.4 prices the norms at O(nd) (one streaming read of
// A, HBM-bound) and TopK as a light vector operation (d scores, latency-bound).
//
// colnorm_partial: one 16-byte load per thread per row (8 bf16 or 4 fp32
//   columns); a wave covers up to 1 KB of a row, so every row segment is read
//   with full cache lines.  Each workgroup sums a chunk of rows for one strip
//   of columns in fp32, combines its row-lanes through LDS in a fixed order
//   and writes one partial per column.  No atomics: the result is
//   bit-reproducible.
// colnorm_finalize: adds the row-chunk partials in ascending chunk order and
//   takes a correctly rounded square root.
// select: one workgroup per score vector.  Three LDS histogram passes over
//   11/11/10-bit digits of an order-preserving key find the exact k-th
//   largest key T; a block-wide scan then keeps, in ascending index order,
//   every key above T and the lowest-indexed keys equal to T.
#include "rmm_internal.h"

namespace rmm {

namespace {

constexpr int kNormThreads = 256;

template <typename T>
struct Vec16;  // one 16-byte load
template <>
struct Vec16<uint16_t> {
    static constexpr int N = 8;
    __device__ static void load(const uint16_t *p, float (&v)[8]) {
        uint4 q = *reinterpret_cast<const uint4 *>(p);
        uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    __device__ static float scalar(const uint16_t *p) { return bf16_to_f32(*p); }
};
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void load(const float *p, float (&v)[4]) {
        float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    }
    __device__ static float scalar(const float *p) { return *p; }
};

// grid: (strips, chunks, batch); block: kNormThreads = tc column-lanes x tr row-lanes.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void colnorm_partial_kernel(const T *__restrict__ A, int64_t n, int64_t d,
                                                                       int64_t lda, int64_t strideA, int tc,
                                                                       int64_t rows_per_chunk, int vec_ok,
                                                                       float *__restrict__ part) {
    constexpr int V = Vec16<T>::N;
    __shared__ float red[kNormThreads * V];
    const int tid = threadIdx.x;
    const int tx = tid % tc, ty = tid / tc, tr = kNormThreads / tc;
    const int64_t b = blockIdx.z;
    const int64_t j0 = (int64_t)blockIdx.x * tc * V + (int64_t)tx * V;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = min(n, r0 + rows_per_chunk);
    const T *Ab = A + b * strideA;

    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;

    if (vec_ok && j0 + V <= d) {
        const T *p = Ab + j0;
        int64_t i = r0 + ty;
        // four rows in flight per iteration; each row's sum still runs in row order
        for (; i + 3 * tr < r1; i += 4 * tr) {
            float v0[V], v1[V], v2[V], v3[V];
            Vec16<T>::load(p + i * lda, v0);
            Vec16<T>::load(p + (i + tr) * lda, v1);
            Vec16<T>::load(p + (i + 2 * tr) * lda, v2);
            Vec16<T>::load(p + (i + 3 * tr) * lda, v3);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                acc[e] = fmaf(v0[e], v0[e], acc[e]);
                acc[e] = fmaf(v1[e], v1[e], acc[e]);
                acc[e] = fmaf(v2[e], v2[e], acc[e]);
                acc[e] = fmaf(v3[e], v3[e], acc[e]);
            }
        }
        for (; i < r1; i += tr) {
            float v0[V];
            Vec16<T>::load(p + i * lda, v0);
#pragma unroll
            for (int e = 0; e < V; ++e) acc[e] = fmaf(v0[e], v0[e], acc[e]);
        }
    } else {
        for (int64_t i = r0 + ty; i < r1; i += tr) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if (j0 + e < d) {
                    float x = Vec16<T>::scalar(Ab + i * lda + j0 + e);
                    acc[e] = fmaf(x, x, acc[e]);
                }
            }
        }
    }

#pragma unroll
    for (int e = 0; e < V; ++e) red[ty * tc * V + tx * V + e] = acc[e];
    __syncthreads();
    // row-lanes are combined in ascending order by the first tc*V threads
    const int cols = tc * V;
    for (int c = tid; c < cols; c += kNormThreads) {
        float sum = 0.f;
        for (int y = 0; y < tr; ++y) sum += red[y * cols + c];
        int64_t j = (int64_t)blockIdx.x * cols + c;
        if (j < d) part[(b * gridDim.y + blockIdx.y) * d + j] = sum;
    }
}

__global__ __launch_bounds__(256) void colnorm_finalize_kernel(const float *__restrict__ part, int64_t chunks,
                                                               int64_t d, int64_t total, float *__restrict__ s) {
    int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= total) return;
    int64_t b = q / d, j = q - b * d;
    const float *p = part + b * chunks * d + j;
    float sum = 0.f;
    for (int64_t r = 0; r < chunks; ++r) sum += p[r * d];
    s[q] = __fsqrt_rn(sum);
}

// ------------------------------------------------------------------ block scan
template <int BS>
__device__ __forceinline__ int block_exclusive_scan(int v, int *sm, int &total) {
    constexpr int NW = BS / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sm[w] = x;
    __syncthreads();
    if (w == 0) {
        int t = lane < NW ? sm[lane] : 0;
        int u = t;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            int y = __shfl_up(u, o, 64);
            if (lane >= o) u += y;
        }
        if (lane < NW) sm[lane] = u - t;
        if (lane == NW - 1) sm[NW] = u;
    }
    __syncthreads();
    int res = sm[w] + x - v;
    total = sm[NW];
    __syncthreads();
    return res;
}

struct KeySource {
    const float *s;     // scores, or
    const void *a;      // a single activation row (decode): score = |a_j|
    int a_bf16;
    const uint32_t *lds;  // keys staged in LDS (may be null)

    __device__ __forceinline__ float score(int64_t j) const {
        if (s) return s[j];
        float x = a_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(a)[j]) : static_cast<const float *>(a)[j];
        return fabsf(x);
    }
    __device__ __forceinline__ uint32_t key(int64_t j) const { return lds ? lds[j] : score_key(score(j)); }
};

// grid: batch; block: BS.  dynamic LDS: d keys when use_lds.
template <int BS>
__global__ __launch_bounds__(BS) void select_kernel(const float *__restrict__ s_all, const void *__restrict__ a_all,
                                                     int a_bf16, int64_t a_stride, int64_t d, int64_t k,
                                                     int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                     float *__restrict__ aval, int use_lds) {
    extern __shared__ uint32_t keys[];
    __shared__ int hist[2048];
    __shared__ int scan_sm[BS / 64 + 1];
    __shared__ int found[2];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;

    KeySource src;
    src.s = s_all ? s_all + b * d : nullptr;
    src.a = a_all ? (a_bf16 ? (const void *)(static_cast<const uint16_t *>(a_all) + b * a_stride)
                            : (const void *)(static_cast<const float *>(a_all) + b * a_stride))
                  : nullptr;
    src.a_bf16 = a_bf16;
    src.lds = nullptr;
    if (use_lds) {
        for (int64_t j = tid; j < d; j += BS) keys[j] = score_key(src.score(j));
        src.lds = keys;
        __syncthreads();
    }

    // ---- radix select of the k-th largest key: digits [31:21], [20:10], [9:0]
    uint32_t prefix = 0, pmask = 0;
    int rem = (int)k;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int p = 0; p < 3; ++p) {
        const int sh = shifts[p];
        const uint32_t dmask = (1u << widths[p]) - 1u;
        for (int q = tid; q < 2048; q += BS) hist[q] = 0;
        __syncthreads();
        for (int64_t j = tid; j < d; j += BS) {
            uint32_t key = src.key(j);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dmask], 1);
        }
        __syncthreads();
        // thread t owns bins from the top: 2047 - (t*NB + e)
        constexpr int NB = 2048 / BS;
        int c = 0;
#pragma unroll
        for (int e = 0; e < NB; ++e) c += hist[2047 - (tid * NB + e)];
        int total;
        int before = block_exclusive_scan<BS>(c, scan_sm, total);
        if (before < rem && before + c >= rem) {
            int cum = before;
#pragma unroll
            for (int e = 0; e < NB; ++e) {
                int bin = 2047 - (tid * NB + e);
                int h = hist[bin];
                if (cum + h >= rem) {
                    found[0] = bin;
                    found[1] = rem - cum;
                    break;
                }
                cum += h;
            }
        }
        __syncthreads();
        prefix |= uint32_t(found[0]) << sh;
        pmask |= dmask << sh;
        rem = found[1];
        __syncthreads();
    }
    const uint32_t T = prefix;  // exact k-th largest key; take `rem` of the keys equal to it

    // ---- ascending compaction over contiguous per-thread segments
    const int64_t E = (d + BS - 1) / BS;
    const int64_t j0 = min(d, (int64_t)tid * E), j1 = min(d, j0 + E);
    int eq = 0;
    for (int64_t j = j0; j < j1; ++j) eq += (src.key(j) == T);
    int tot;
    int eq_before = block_exclusive_scan<BS>(eq, scan_sm, tot);
    int sel = 0;
    {
        int e = eq_before;
        for (int64_t j = j0; j < j1; ++j) {
            uint32_t key = src.key(j);
            if (key > T) ++sel;
            else if (key == T) {
                if (e < rem) ++sel;
                ++e;
            }
        }
    }
    int pos = block_exclusive_scan<BS>(sel, scan_sm, tot);
    int32_t *idx = idx_all + b * ld_idx;
    {
        int e = eq_before;
        for (int64_t j = j0; j < j1; ++j) {
            uint32_t key = src.key(j);
            bool take = key > T;
            if (key == T) {
                take = e < rem;
                ++e;
            }
            if (take && pos < k) {
                idx[pos] = (int32_t)j;
                if (aval) {
                    float x = src.a_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(src.a)[j])
                                         : static_cast<const float *>(src.a)[j];
                    aval[b * k + pos] = x;
                }
                ++pos;
            }
        }
    }
}

__global__ void iota_kernel(int32_t *idx, int64_t k, int64_t total) {
    int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < total) idx[q] = (int32_t)(q % k);
}

unsigned g_select_attr_done = 0;  // bit per device

}  // namespace

ColnormPlan colnorm_plan(rmm_dtype_t dt, int64_t n, int64_t d, int64_t batch) {
    const int V = dt == RMM_BF16 ? 8 : 4;
    int tc = 64;
    while (tc > 1 && (int64_t)tc * V / 2 >= d) tc /= 2;
    const int tr = kNormThreads / tc;
    ColnormPlan p;
    p.tc = tc;
    p.strips = (int)((d + (int64_t)tc * V - 1) / ((int64_t)tc * V));
    // about 512 workgroups, each thread summing at least 8 rows
    int64_t want = (512 + (int64_t)p.strips * batch - 1) / ((int64_t)p.strips * batch);
    int64_t max_chunks = (n + 8 * tr - 1) / (8 * tr);
    int64_t chunks = want < max_chunks ? want : max_chunks;
    if (chunks < 1) chunks = 1;
    p.rows_per_chunk = (n + chunks - 1) / chunks;
    p.chunks = (int)((n + p.rows_per_chunk - 1) / p.rows_per_chunk);
    return p;
}

hipError_t launch_colnorm_partial(const void *A, rmm_dtype_t dt, int64_t n, int64_t d, int64_t lda, int64_t batch,
                                  int64_t strideA, const ColnormPlan &p, float *part, hipStream_t stream) {
    dim3 grid(p.strips, p.chunks, (unsigned)batch);
    const int esz = dt == RMM_BF16 ? 2 : 4;
    const int V = 16 / esz;
    const int vec_ok = ((uintptr_t)A % 16 == 0) && (lda % V == 0) && (batch == 1 || strideA % V == 0);
    if (dt == RMM_BF16)
        colnorm_partial_kernel<uint16_t><<<grid, kNormThreads, 0, stream>>>(
            static_cast<const uint16_t *>(A), n, d, lda, strideA, p.tc, p.rows_per_chunk, vec_ok, part);
    else
        colnorm_partial_kernel<float><<<grid, kNormThreads, 0, stream>>>(
            static_cast<const float *>(A), n, d, lda, strideA, p.tc, p.rows_per_chunk, vec_ok, part);
    return hipGetLastError();
}

hipError_t launch_colnorm_finalize(const float *part, int64_t chunks, int64_t d, int64_t batch, float *s,
                                   hipStream_t stream) {
    int64_t total = d * batch;
    colnorm_finalize_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(part, chunks, d, total, s);
    return hipGetLastError();
}

// Scores are staged in LDS when they fit comfortably (d <= 24576 keys, 96 KB).
static constexpr int64_t kSelectLdsKeys = 24576;

hipError_t launch_select(const float *s, const void *a_src, rmm_dtype_t a_dt, int64_t a_stride, int64_t batch,
                         int64_t d, int64_t k, int32_t *idx, int64_t ld_idx, float *aval, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (dev < 32 && !(g_select_attr_done & (1u << dev))) {
        hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<1024>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kSelectLdsKeys * 4));
        hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_kernel<256>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kSelectLdsKeys * 4));
        if (e1 != hipSuccess) return e1;
        if (e2 != hipSuccess) return e2;
        g_select_attr_done |= 1u << dev;
    }
    const int use_lds = d <= kSelectLdsKeys;
    const size_t lds = use_lds ? (size_t)d * 4 : 0;
    const int a_bf16 = a_dt == RMM_BF16;
    if (d > 2048)
        select_kernel<1024><<<(unsigned)batch, 1024, lds, stream>>>(s, a_src, a_bf16, a_stride, d, k, idx, ld_idx,
                                                                   aval, use_lds);
    else
        select_kernel<256><<<(unsigned)batch, 256, lds, stream>>>(s, a_src, a_bf16, a_stride, d, k, idx, ld_idx,
                                                                 aval, use_lds);
    return hipGetLastError();
}

hipError_t launch_iota(int32_t *idx, int64_t k, int64_t batch, hipStream_t stream) {
    int64_t total = k * batch;
    iota_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(idx, k, total);
    return hipGetLastError();
}

}  // namespace rmm
