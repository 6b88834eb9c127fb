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
        // eight rows in flight per iteration; each column's sum still runs in row order
        for (; i + 7 * tr < r1; i += 8 * tr) {
            float v[8][V];
#pragma unroll
            for (int q = 0; q < 8; ++q) Vec16<T>::load(p + (i + q * tr) * lda, v[q]);
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int e = 0; e < V; ++e) acc[e] = fmaf(v[q][e], v[q][e], acc[e]);
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

// 64 columns per workgroup; four row-chunk groups per column, each summing
// every fourth chunk in ascending order (four loads in flight), then combined
// as ((g0 + g1) + g2) + g3.
__global__ __launch_bounds__(256) void colnorm_finalize_kernel(const float *__restrict__ part, int64_t chunks,
                                                               int64_t d, float *__restrict__ s) {
    __shared__ float red[4][64];
    const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 64 + c;
    float sum = 0.f;
    if (j < d) {
        const float *p = part + b * chunks * d + j;
        int64_t r = g;
        for (; r + 12 < chunks; r += 16) {
            const float v0 = p[r * d], v1 = p[(r + 4) * d], v2 = p[(r + 8) * d], v3 = p[(r + 12) * d];
            sum += v0;
            sum += v1;
            sum += v2;
            sum += v3;
        }
        for (; r < chunks; r += 4) sum += p[r * d];
    }
    red[g][c] = sum;
    __syncthreads();
    if (g == 0 && j < d) s[b * d + j] = __fsqrt_rn(((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]);
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

// Long score vectors (beyond the register-resident kernel's reach): keys are
// re-read from LDS (or global memory when d is very large) in every pass.
// grid: batch; block: BS.  dynamic LDS: d keys when use_lds.
template <int BS>
__global__ __launch_bounds__(BS) void select_big_kernel(const float *__restrict__ s_all, const void *__restrict__ a_all,
                                                        int a_bf16, int64_t a_stride, int64_t d, int64_t k,
                                                        int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                        int32_t *__restrict__ pad_all, int64_t ld_pad,
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
    int32_t *idx = idx_all ? idx_all + b * ld_idx : nullptr;
    int32_t *pad = pad_all ? pad_all + b * ld_pad : nullptr;
    if (pad)
        for (int64_t q = k + tid; q < ld_pad; q += BS) pad[q] = -1;
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
                if (idx) idx[pos] = (int32_t)j;
                if (pad) pad[pos] = (int32_t)j;
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

// Register-resident exact TopK for d <= BS * E: thread t owns the contiguous
// scores [t*E, t*E + E).  Three radix passes over 11/11/10-bit digits of the
// order-preserving key, each: LDS histogram (ping-pong buffers, so the next
// one is cleared while this one fills), per-thread bin sums from the top, a
// wave scan plus wave totals to find the digit holding the k-th largest key.
// The passes stop early once the digit's bin holds exactly the keys still
// needed.  Compaction in ascending index order keeps every key whose resolved
// prefix is larger and the lowest-indexed keys whose prefix equals it.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

template <int BS, int E>
__global__ __launch_bounds__(BS) void select_reg_kernel(const float *__restrict__ s_all, const void *__restrict__ a_all,
                                                        int a_bf16, int64_t a_stride, int d, int k,
                                                        int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                        int32_t *__restrict__ pad_all, int64_t ld_pad,
                                                        float *__restrict__ aval) {
    constexpr int NW = BS / 64;
    constexpr int NB = 2048 / BS;
    __shared__ int hist[2][2048];
    __shared__ int wsum[5][NW];
    __shared__ int found[3][3];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t b = blockIdx.x;

    KeySource src;
    src.s = s_all ? s_all + b * d : nullptr;
    src.a = a_all ? (a_bf16 ? (const void *)(static_cast<const uint16_t *>(a_all) + b * a_stride)
                            : (const void *)(static_cast<const float *>(a_all) + b * a_stride))
                  : nullptr;
    src.a_bf16 = a_bf16;
    src.lds = nullptr;

    const int j0 = tid * E;
    const int nv = max(0, min(E, d - j0));
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = e < nv ? score_key(src.score(j0 + e)) : 0u;

    for (int q = tid; q < 2048; q += BS) hist[0][q] = 0;
    __syncthreads();

    uint32_t prefix = 0, pmask = 0;
    int rem = k;
    const int shifts[3] = {21, 10, 0};
    const uint32_t dmasks[3] = {0x7ffu, 0x7ffu, 0x3ffu};
#pragma unroll 1
    for (int p = 0; p < 3; ++p) {
        int *H = hist[p & 1];
        if (p < 2)
            for (int q = tid; q < 2048; q += BS) hist[(p + 1) & 1][q] = 0;
        const int sh = shifts[p];
        const uint32_t dm = dmasks[p];
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (e < nv && (key[e] & pmask) == prefix) atomicAdd(&H[(key[e] >> sh) & dm], 1);
        __syncthreads();
        int c = 0;
#pragma unroll
        for (int e = 0; e < NB; ++e) c += H[2047 - (tid * NB + e)];
        const int incl = wave_incl_scan(c);
        if (lane == 63) wsum[p][w] = incl;
        __syncthreads();
        int before = incl - c;
        for (int v = 0; v < w; ++v) before += wsum[p][v];
        if (before < rem && before + c >= rem) {
            int cum = before;
            for (int e = 0; e < NB; ++e) {
                const int bin = 2047 - (tid * NB + e);
                const int h = H[bin];
                if (cum + h >= rem) {
                    found[p][0] = bin;
                    found[p][1] = rem - cum;
                    found[p][2] = h;
                    break;
                }
                cum += h;
            }
        }
        __syncthreads();
        prefix |= uint32_t(found[p][0]) << sh;
        pmask |= dm << sh;
        rem = found[p][1];
        if (found[p][2] == rem) break;  // every key left in this bin is kept
    }

    // compaction: masked key above prefix -> kept; equal -> first `rem` by index
    int eq = 0, gt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e < nv) {
            const uint32_t mk = key[e] & pmask;
            eq += mk == prefix;
            gt += mk > prefix;
        }
    }
    int incl = wave_incl_scan(eq);
    if (lane == 63) wsum[3][w] = incl;
    __syncthreads();
    int eqb = incl - eq;
    for (int v = 0; v < w; ++v) eqb += wsum[3][v];
    const int sel = gt + max(0, min(eq, rem - eqb));
    incl = wave_incl_scan(sel);
    if (lane == 63) wsum[4][w] = incl;
    __syncthreads();
    int pos = incl - sel;
    for (int v = 0; v < w; ++v) pos += wsum[4][v];

    int32_t *idx = idx_all ? idx_all + b * ld_idx : nullptr;
    int32_t *pad = pad_all ? pad_all + b * ld_pad : nullptr;
    if (pad)
        for (int64_t q = k + tid; q < ld_pad; q += BS) pad[q] = -1;
    int er = eqb;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (e < nv) {
            const uint32_t mk = key[e] & pmask;
            bool take = mk > prefix;
            if (mk == prefix) {
                take = er < rem;
                ++er;
            }
            if (take && pos < k) {
                const int j = j0 + e;
                if (idx) idx[pos] = j;
                if (pad) pad[pos] = j;
                if (aval) {
                    aval[b * k + pos] = src.a_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(src.a)[j])
                                                   : static_cast<const float *>(src.a)[j];
                }
                ++pos;
            }
        }
    }
}

__global__ void iota_kernel(int32_t *idx, int64_t k, int64_t ld, int64_t total) {
    int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < total) {
        const int64_t t = q % ld;
        idx[q] = t < k ? (int32_t)t : -1;
    }
}

unsigned g_select_attr_done = 0;  // bit per device

}  // namespace

// Strips of 16 threads x one 16-byte load (128 bf16 / 64 fp32 columns: one
// 256-byte segment per row) and about 1024 workgroups, each thread summing at
// least 8 rows: the fastest shape measured on MI355X for the 4096 x 4096 bf16
// activation block (7.4 us, 4.6 TB/s, against 13-15 us for 512-column strips).
ColnormPlan colnorm_plan(rmm_dtype_t dt, int64_t n, int64_t d, int64_t batch) {
    const int V = dt == RMM_BF16 ? 8 : 4;
    int tc = 16;
    while (tc > 1 && (int64_t)tc * V / 2 >= d) tc /= 2;
    const int tr = kNormThreads / tc;
    ColnormPlan p;
    p.tc = tc;
    p.strips = (int)((d + (int64_t)tc * V - 1) / ((int64_t)tc * V));
    int64_t want = (1024 + (int64_t)p.strips * batch - 1) / ((int64_t)p.strips * batch);
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
    dim3 grid((unsigned)((d + 63) / 64), (unsigned)batch);
    colnorm_finalize_kernel<<<grid, 256, 0, stream>>>(part, chunks, d, s);
    return hipGetLastError();
}

// Scores are staged in LDS when they fit comfortably (d <= 24576 keys, 96 KB).
static constexpr int64_t kSelectLdsKeys = 24576;

hipError_t launch_select(const float *s, const void *a_src, rmm_dtype_t a_dt, int64_t a_stride, int64_t batch,
                         int64_t d, int64_t k, int32_t *idx, int64_t ld_idx, int32_t *idx_pad, int64_t ld_pad,
                         float *aval, hipStream_t stream) {
    const int a_bf16 = a_dt == RMM_BF16;
    const unsigned g = (unsigned)batch;
    if (d <= 256) {
        select_reg_kernel<64, 4><<<g, 64, 0, stream>>>(s, a_src, a_bf16, a_stride, (int)d, (int)k, idx, ld_idx,
                                                       idx_pad, ld_pad, aval);
    } else if (d <= 4096) {
        select_reg_kernel<256, 16><<<g, 256, 0, stream>>>(s, a_src, a_bf16, a_stride, (int)d, (int)k, idx, ld_idx,
                                                          idx_pad, ld_pad, aval);
    } else if (d <= 8192) {
        select_reg_kernel<512, 16><<<g, 512, 0, stream>>>(s, a_src, a_bf16, a_stride, (int)d, (int)k, idx, ld_idx,
                                                          idx_pad, ld_pad, aval);
    } else if (d <= 16384) {
        select_reg_kernel<1024, 16><<<g, 1024, 0, stream>>>(s, a_src, a_bf16, a_stride, (int)d, (int)k, idx,
                                                            ld_idx, idx_pad, ld_pad, aval);
    } else {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
        if (dev < 32 && !(g_select_attr_done & (1u << dev))) {
            hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void *>(&select_big_kernel<1024>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                (int)(kSelectLdsKeys * 4));
            if (e1 != hipSuccess) return e1;
            g_select_attr_done |= 1u << dev;
        }
        const int use_lds = d <= kSelectLdsKeys;
        const size_t lds = use_lds ? (size_t)d * 4 : 0;
        select_big_kernel<1024><<<g, 1024, lds, stream>>>(s, a_src, a_bf16, a_stride, d, k, idx, ld_idx, idx_pad,
                                                          ld_pad, aval, use_lds);
    }
    return hipGetLastError();
}

hipError_t launch_iota(int32_t *idx, int64_t k, int64_t ld, int64_t batch, hipStream_t stream) {
    int64_t total = ld * batch;
    iota_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(idx, k, ld, total);
    return hipGetLastError();
}

}  // namespace rmm
