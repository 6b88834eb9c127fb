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

// bf16 column sums of squares with every load of a thread issued up front:
// thread (tx, ty) of a 256-thread workgroup owns eight columns and RPT rows
// (ty, ty + tr, ...) of its strip x chunk; all RPT 16-byte loads are in
// flight before the first multiply, so one memory round trip covers the
// whole workgroup.  Rows past the chunk or past n read as zero (raw buffer
// loads with an out-of-range offset).  Each column's sum still runs in row
// order within a thread, then over row lanes in order through LDS.
template <int RPT>
__global__ __launch_bounds__(kNormThreads) void colnorm_rows_kernel(const uint16_t *__restrict__ A, int64_t n,
                                                                    int64_t d, int64_t lda, int64_t strideA, int tc,
                                                                    int64_t rows_per_chunk, int64_t a_bytes,
                                                                    float *__restrict__ part) {
    __shared__ float red[kNormThreads * 8];
    const int tid = threadIdx.x;
    const int tx = tid % tc, ty = tid / tc, tr = kNormThreads / tc;
    const int64_t b = blockIdx.z;
    const int64_t j0 = (int64_t)blockIdx.x * tc * 8 + (int64_t)tx * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = min(n, r0 + rows_per_chunk);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(A + b * strideA), (short)0, (int)a_bytes, 0x00020000);

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (j0 + 8 <= d) {  // d % 8 == 0 on this path
        uint4 v[RPT];
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int64_t i = r0 + ty + (int64_t)q * tr;
            const uint32_t off = i < r1 ? (uint32_t)((i * lda + j0) * 2) : 0x80000000u;
            v[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        }
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float lo = __uint_as_float(w[h] << 16), hi = __uint_as_float(w[h] & 0xffff0000u);
                acc[2 * h] = fmaf(lo, lo, acc[2 * h]);
                acc[2 * h + 1] = fmaf(hi, hi, acc[2 * h + 1]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[ty * tc * 8 + tx * 8 + e] = acc[e];
    __syncthreads();
    const int cols = tc * 8;
    for (int c = tid; c < cols; c += kNormThreads) {
        float sum = 0.f;
        for (int y = 0; y < tr; ++y) sum += red[y * cols + c];
        const int64_t j = (int64_t)blockIdx.x * cols + c;
        if (j < d) part[(b * gridDim.y + blockIdx.y) * d + j] = sum;
    }
}

// bf16 column sums of squares that also write the transposed copy At (d x n,
// rows ldt apart) of the block: the gather source of the two-operand GEMM,
// whose kept rows At[I_t, :] are then contiguous like the rows of B.  The
// pass reads A once and writes it once, both in long row runs.  A workgroup
// takes a TC-column strip and a chunk of rows and walks the chunk in TR-row
// tiles.  A tile is loaded in 2*TC-byte row runs (16 bytes a lane), its
// squares are summed per lane, and it is stored to LDS; after one barrier
// each lane reads back an 8 x 8 block (eight 16-byte reads), transposes it
// with byte permutes and writes it as one 16-byte piece of each of eight rows
// of At, the lanes of a wave forming 2*TR-byte runs.  The next tile's loads
// go out right after the barrier and land while the current tile is
// transposed and written; two LDS buffers leave one barrier per tile.  The
// 16-byte slots of a row are XOR-swizzled by its 8-row block, so the row
// writes and the block reads both spread over the LDS banks.  Squares are
// summed per lane in row order, then over the lanes and waves that share a
// column in a fixed order: the partial of a column and chunk has a fixed
// summation order.  n % 8 == 0 and d % 8 == 0, so a 16-byte piece or an
// 8 x 8 block lies wholly inside or wholly outside the block.
template <int TC, int TR, int NT>
__global__ __launch_bounds__(NT) void colnorm_transpose_kernel(const uint16_t *__restrict__ A, int64_t n,
                                                                        int64_t d, int64_t lda,
                                                                        int64_t rows_per_chunk, int64_t a_bytes,
                                                                        uint16_t *__restrict__ At, int64_t ldt,
                                                                        float *__restrict__ part) {
    constexpr int CPR = TC / 8;                       // 16-byte pieces per tile row
    constexpr int RPL = NT / CPR;           // tile rows per round of loads
    constexpr int NL = TR / RPL;                      // loads per lane per tile
    constexpr int RB = TR / 8;                        // 8-row blocks per tile
    constexpr int NB = (TC / 8) * RB / NT;  // 8 x 8 blocks per lane per tile
    constexpr int NW = NT / 64;
    static_assert(NL >= 1 && NB >= 1 && (CPR & (CPR - 1)) == 0 && CPR <= 64 && TR % RPL == 0, "tile shape");
    __shared__ uint4 buf[2][TR * CPR];
    __shared__ float red[NW][TC];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lc = tid % CPR, lr = tid / CPR;
    const int64_t c0 = (int64_t)blockIdx.x * TC;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = min(n, r0 + rows_per_chunk);
    const int ntiles = (int)((r1 - r0 + TR - 1) / TR);
    const int64_t lcol = c0 + 8 * lc;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(A), (short)0, (int)a_bytes, 0x00020000);
    uint4 v[NL];
    // rows past the chunk end (and columns past d) read as zero, with no traffic
    auto load_tile = [&](int t) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int64_t row = r0 + (int64_t)t * TR + lr + RPL * j;
            const uint32_t off = (row < r1 && lcol < d) ? (uint32_t)((row * lda + lcol) * 2) : 0x80000000u;
            v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        }
    };
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        uint4 *b = buf[t & 1];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const uint32_t wv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float lo = __uint_as_float(wv[h] << 16), hi = __uint_as_float(wv[h] & 0xffff0000u);
                acc[2 * h] = fmaf(lo, lo, acc[2 * h]);
                acc[2 * h + 1] = fmaf(hi, hi, acc[2 * h + 1]);
            }
            const int r = lr + RPL * j;
            b[r * CPR + (lc ^ ((r >> 3) & (CPR - 1)))] = v[j];
        }
        __syncthreads();
        load_tile(t + 1);
        const int64_t tr0 = r0 + (int64_t)t * TR;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int blk = tid + q * NT;
            const int rb = blk % RB, cb = blk / RB;
            uint32_t wd[8][4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 x = b[(8 * rb + i) * CPR + (cb ^ (rb & (CPR - 1)))];
                wd[i][0] = x.x;
                wd[i][1] = x.y;
                wd[i][2] = x.z;
                wd[i][3] = x.w;
            }
            const int64_t row = tr0 + 8 * rb, col = c0 + 8 * cb;
            if (row < r1 && col < d) {
                // column e of the block: the low (e even) or high (e odd)
                // halves of word e / 2 of rows 0..7, paired into four words
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    uint4 o;
                    o.x = __builtin_amdgcn_perm(wd[1][e >> 1], wd[0][e >> 1], sel);
                    o.y = __builtin_amdgcn_perm(wd[3][e >> 1], wd[2][e >> 1], sel);
                    o.z = __builtin_amdgcn_perm(wd[5][e >> 1], wd[4][e >> 1], sel);
                    o.w = __builtin_amdgcn_perm(wd[7][e >> 1], wd[6][e >> 1], sel);
                    *reinterpret_cast<uint4 *>(At + (col + e) * ldt + row) = o;
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float x = acc[e];
#pragma unroll
        for (int o = CPR; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
        acc[e] = x;
    }
    if (lane < CPR) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[w][8 * lc + e] = acc[e];
    }
    __syncthreads();
    for (int c = tid; c < TC; c += NT) {
        if (c0 + c < d) {
            float sum = red[0][c];
#pragma unroll
            for (int y = 1; y < NW; ++y) sum += red[y][c];
            part[(int64_t)blockIdx.y * d + c0 + c] = sum;
        }
    }
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

// ------------------------------------------------------------------ caller-supplied index set
// Block-wide exclusive maximum (identity -1) of one int per thread.
template <int BS>
__device__ __forceinline__ int block_exclusive_max(int v, int *sm, int &total) {
    constexpr int NW = BS / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x = max(x, y);
    }
    if (lane == 63) sm[w] = x;
    __syncthreads();
    if (w == 0) {
        const int t = lane < NW ? sm[lane] : -1;
        int u = t;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const int y = __shfl_up(u, o, 64);
            if (lane >= o) u = max(u, y);
        }
        const int ex = __shfl_up(u, 1, 64);
        if (lane < NW) sm[lane] = lane == 0 ? -1 : ex;
        if (lane == NW - 1) sm[NW] = u;
    }
    __syncthreads();
    const int below = __shfl_up(x, 1, 64);
    const int res = max(sm[w], lane == 0 ? -1 : below);
    total = sm[NW];
    __syncthreads();
    return res;
}

// A caller-supplied kept set (the static variant of the selection: the same
// I reused across calls) turned into the padded list the gather kernels
// read.  Entry t of row b is kept when it lies in [0, d) and exceeds every
// earlier in-range entry of the row, so the kept entries are strictly
// ascending whatever the input; they are compacted to the front and the
// rest of the ld_pad slots are -1.  For a decode row (a_row given) the kept
// values a[I_t] go to aval, and the slots from the kept count up to k read
// row 0 with value 0 instead of -1 (the GEMV reads k slots).  One workgroup
// per row; the k entries are taken in segments of BS * EP.
template <int BS, int EP>
__global__ __launch_bounds__(BS) void index_prepare_kernel(const int32_t *__restrict__ idx_all, int64_t k, int64_t d,
                                                           int32_t *__restrict__ pad_all, int64_t ld_pad,
                                                           const uint16_t *__restrict__ a_row,
                                                           float *__restrict__ aval) {
    __shared__ int sm[BS / 64 + 1];
    const int64_t b = blockIdx.x;
    const int32_t *idx = idx_all + b * k;
    int32_t *pad = pad_all + b * ld_pad;
    int carry_max = -1, carry_pos = 0;
    for (int64_t s0 = 0; s0 < k; s0 += (int64_t)BS * EP) {
        const int64_t j0 = s0 + (int64_t)threadIdx.x * EP;
        int32_t v[EP];
        int tmax = -1;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            v[e] = j0 + e < k ? idx[j0 + e] : -1;
            if (v[e] >= 0 && v[e] < d) tmax = max(tmax, v[e]);
        }
        int seg_max;
        const int before = max(carry_max, block_exclusive_max<BS>(tmax, sm, seg_max));
        int run = before, cnt = 0;
        bool keep[EP];
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            const bool in = v[e] >= 0 && v[e] < d;
            keep[e] = in && v[e] > run;
            if (in) run = max(run, v[e]);
            cnt += keep[e];
        }
        int seg_cnt;
        int pos = carry_pos + block_exclusive_scan<BS>(cnt, sm, seg_cnt);
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            if (keep[e]) {
                pad[pos] = v[e];
                if (aval) aval[b * k + pos] = bf16_to_f32(a_row[v[e]]);
                ++pos;
            }
        }
        carry_max = max(carry_max, seg_max);
        carry_pos += seg_cnt;
    }
    for (int64_t q = carry_pos + threadIdx.x; q < ld_pad; q += BS) {
        const bool gemv_slot = aval && q < k;
        pad[q] = gemv_slot ? 0 : -1;
        if (gemv_slot) aval[b * k + q] = 0.f;
    }
}

// ------------------------------------------------------------------ wave helpers (DPP)
// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane
// row (row_shr 1, 2, 4, 8), then row broadcasts of lane 15 and lane 31.
__device__ __forceinline__ int wave_incl_add(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
    return x;
}
// Maximum over the wave (same shift pattern; lane 63 holds the result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

template <int BS>
struct SelectShared {
    int hist[2][2048];
    int wsum[4][BS / 64];
    uint32_t wmax[2][BS / 64];
    uint32_t wlow[BS / 64];
    int found[4][3];
};

// Bitwise OR over the wave (lane 63 holds the result).
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t x) {
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
    return x;
}

// Exact TopK of the keys held by a workgroup: thread t owns keys
// [t*E, t*E + nv) (nv <= E, order-preserving keys of the scores).  Keeps the
// k largest, ties to the lower index, and writes them in ascending order to
// idx (when given), pad (when given; entries k..ld_pad-1 become -1) and, for
// a decode row, their activation values to aval.
//  * min and max of the keys fix the highest bit where keys differ, so the
//    first 11-bit radix digit starts there and spreads the keys over the 2048
//    LDS bins (no pile-up of atomics on a few bins);
//  * each pass: histogram (ping-pong buffers: the next one is cleared while
//    this one fills), per-thread bin sums from the top, DPP wave scan plus
//    wave totals locate the bin holding the k-th largest key; passes stop
//    once that bin holds exactly the keys still needed;
//  * compaction: one packed block scan of (larger, equal) counts gives each
//    thread its output position and the number of equal keys before it.
template <int BS, int E>
__device__ void block_select(SelectShared<BS> &sh, const uint32_t (&key)[E], int nv, int j0, int k,
                             int32_t *__restrict__ idx, int32_t *__restrict__ pad, int64_t ld_pad,
                             float *__restrict__ aval, const float (&vals)[E], int32_t *out_idx,
                             float *out_val) {
    constexpr int NW = BS / 64;
    constexpr int NB = 2048 / BS;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    // extent of the keys: max, min, and the lowest bit any key has set (bits
    // below it are zero in every key and never need resolving; bf16 scores
    // leave the low 16 bits clear)
    uint32_t kmax = 0u, kmin = 0xffffffffu, kor = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (e < nv) {
            kmax = max(kmax, key[e]);
            kmin = min(kmin, key[e]);
            kor |= key[e];
        }
    // the cross-lane reductions run with every lane active; only the stores are lane 0's
    kmax = wave_max_u32(kmax);
    kmin = ~wave_max_u32(~kmin);
    kor = (uint32_t)__builtin_amdgcn_readlane((int)wave_or_u32(kor), 63);
    if (lane == 0) {
        sh.wmax[0][w] = kmax;
        sh.wmax[1][w] = ~kmin;
        sh.wlow[w] = kor;
    }
    for (int q = tid; q < 2048; q += BS) sh.hist[0][q] = 0;
    __syncthreads();
    kmax = 0u;
    uint32_t nmin = 0u, allor = 0u;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        kmax = max(kmax, sh.wmax[0][v]);
        nmin = max(nmin, sh.wmax[1][v]);
        allor |= sh.wlow[v];
    }
    kmin = ~nmin;
    const int zbits = allor ? __builtin_ctz(allor) : 0;  // bits below are zero in every key

    uint32_t prefix = kmax, pmask = 0xffffffffu;
    int rem = k;
    if (kmin != kmax) {
        const int hb = 31 - __builtin_clz(kmin ^ kmax);  // highest differing bit
        pmask = hb >= 31 ? 0u : (0xffffffffu << (hb + 1));
        prefix = kmax & pmask;
        int lo = hb + 1;  // bits below `lo` are still unresolved
#pragma unroll 1
        for (int p = 0; lo > zbits; ++p) {
            const int width = lo - zbits >= 11 ? 11 : lo - zbits;
            const int sh_ = lo - width;
            const uint32_t dm = (1u << width) - 1u;
            int *H = sh.hist[p & 1];
            for (int q = tid; q < 2048; q += BS) sh.hist[(p + 1) & 1][q] = 0;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < nv && (key[e] & pmask) == prefix) atomicAdd(&H[(key[e] >> sh_) & dm], 1);
            __syncthreads();
            int c = 0;
#pragma unroll
            for (int e = 0; e < NB; ++e) c += H[2047 - (tid * NB + e)];
            const int incl = wave_incl_add(c);
            if (lane == 63) sh.wsum[p & 1][w] = incl;
            __syncthreads();
            int before = incl - c;
            for (int v = 0; v < w; ++v) before += sh.wsum[p & 1][v];
            if (before < rem && before + c >= rem) {
                int cum = before;
                for (int e = 0; e < NB; ++e) {
                    const int bin = 2047 - (tid * NB + e);
                    const int h = H[bin];
                    if (cum + h >= rem) {
                        sh.found[p & 3][0] = bin;
                        sh.found[p & 3][1] = rem - cum;
                        sh.found[p & 3][2] = h;
                        break;
                    }
                    cum += h;
                }
            }
            __syncthreads();
            prefix |= uint32_t(sh.found[p & 3][0]) << sh_;
            pmask |= dm << sh_;
            rem = sh.found[p & 3][1];
            lo = sh_;
            if (sh.found[p & 3][2] == rem) break;  // every key left in this bin is kept
        }
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
    const int packed = (gt << 16) | eq;  // counts < 2^16 (d <= 16384 on this path)
    const int incl = wave_incl_add(packed);
    if (lane == 63) sh.wsum[2][w] = incl;
    __syncthreads();
    int exclusive = incl - packed;
    for (int v = 0; v < w; ++v) exclusive += sh.wsum[2][v];
    const int gt_before = exclusive >> 16, eq_before = exclusive & 0xffff;
    int pos = gt_before + min(eq_before, rem);
    // the kept indices (and values) land in LDS in output order first, then
    // the whole workgroup copies them out with contiguous stores
    int er = eq_before;
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
                out_idx[pos] = j0 + e;
                if (aval) out_val[pos] = vals[e];
                ++pos;
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < k; q += BS) {
        const int32_t v = out_idx[q];
        if (idx) idx[q] = v;
        if (pad) pad[q] = v;
        if (aval) aval[q] = out_val[q];
    }
    if (pad)
        for (int64_t q = k + tid; q < ld_pad; q += BS) pad[q] = -1;
}

// Raw 32-bit / 16-bit buffer loads (out-of-range offsets read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sel_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int32_t)min(bytes, (int64_t)0x7fffffff), 0x00020000);
}

// Selection per batch entry from a score vector (ROW_BF16 = false: fp32
// scores s) or from a single bf16 activation row (ROW_BF16 = true: score
// |a_j|, the column norm of a one-row block; the kept values a[I_t] go to
// aval).  All loads are issued up front, unconditionally, so their
// latencies overlap.
template <int BS, int E, bool ROW_BF16, bool VEC>
__global__ __launch_bounds__(BS) void select_kernel(const void *__restrict__ src_all, int64_t stride, int d, int k,
                                                    int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                    int32_t *__restrict__ pad_all, int64_t ld_pad,
                                                    float *__restrict__ aval_all) {
    __shared__ SelectShared<BS> sh;
    extern __shared__ int32_t sel_out[];  // k indices, then k values when aval is requested
    const int64_t b = blockIdx.x;
    constexpr int ESZ = ROW_BF16 ? 2 : 4;
    const char *base = static_cast<const char *>(src_all) + b * stride * ESZ;
    const __amdgpu_buffer_rsrc_t r = sel_rsrc(base, (int64_t)d * ESZ);
    const int j0 = threadIdx.x * E;
    const int nv = max(0, min(E, d - j0));
    float vals[E];
    if constexpr (VEC) {
        // E consecutive values per thread in 16-byte pieces (base 16-byte aligned)
        constexpr int PER = 16 / ESZ;
        static_assert(E % PER == 0, "");
#pragma unroll
        for (int q = 0; q < E / PER; ++q) {
            const int p0 = j0 + q * PER;
            uint4 v;
            if (p0 + PER <= d || p0 >= d) {
                v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)p0 * ESZ, 0, 0));
            } else {
                // the piece that holds column d-1 and runs past d: element loads, so that
                // the range check (bytes from d * ESZ on read as zero) never cuts a piece
                uint32_t e[PER];
#pragma unroll
                for (int h = 0; h < PER; ++h) {
                    const uint32_t off = (uint32_t)(p0 + h) * ESZ;
                    if constexpr (ROW_BF16)
                        e[h] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
                    else
                        e[h] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
                }
                if constexpr (ROW_BF16)
                    v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
                else
                    v = make_uint4(e[0], e[1], e[2], e[3]);
            }
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if constexpr (ROW_BF16) {
                    vals[q * PER + 2 * h] = __uint_as_float(w[h] << 16);
                    vals[q * PER + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
                } else {
                    vals[q * PER + h] = __uint_as_float(w[h]);
                }
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t off = (uint32_t)(j0 + e) * ESZ;
            if constexpr (ROW_BF16)
                vals[e] = __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
            else
                vals[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
        }
    }
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = score_key(ROW_BF16 ? fabsf(vals[e]) : vals[e]);
    block_select<BS, E>(sh, key, nv, j0, k, idx_all ? idx_all + b * ld_idx : nullptr,
                        pad_all ? pad_all + b * ld_pad : nullptr, ld_pad, aval_all ? aval_all + b * k : nullptr, vals,
                        sel_out, reinterpret_cast<float *>(sel_out + k));
}

// Norms and selection in one workgroup per batch entry, straight from the
// row-chunk partials: thread t owns columns [t*E, t*E + E), issues every
// partial load of its columns up front (16-byte buffer loads; columns past d
// and chunks past the last read as zero), adds the chunks in ascending order,
// takes the correctly rounded square root and runs block_select on the
// register-resident keys.  This replaces a finalize launch plus a select
// launch when the partials are few (norm_select_ok).
template <int E>
__global__ __launch_bounds__(1024) void norm_select_kernel(const float *__restrict__ part_all, int chunks, int d,
                                                           int k, int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                           int32_t *__restrict__ pad_all, int64_t ld_pad) {
    constexpr int BS = 1024, Q = E / 4, U = 8 / Q;  // 8 loads in flight per thread
    __shared__ SelectShared<BS> sh;
    extern __shared__ int32_t sel_out[];
    const int64_t b = blockIdx.x;
    const float *part = part_all + b * (int64_t)chunks * d;
    const __amdgpu_buffer_rsrc_t r = sel_rsrc(part, (int64_t)chunks * d * 4);
    const int j0 = threadIdx.x * E;
    const int nv = max(0, min(E, d - j0));
    // offsets past the buffer (at most 4 MB here) read as zero; columns past d
    // must not read the next chunk's row, so they and chunks past the last
    // get 2^30 added (both: 2^31), which is out of range
    constexpr uint32_t kFar = 0x40000000u;
    uint32_t base[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) base[q] = j0 + 4 * q < d ? (uint32_t)(j0 + 4 * q) * 4u : kFar;
    float sum[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sum[e] = 0.f;
    for (int c0 = 0; c0 < chunks; c0 += U) {
        uint4 v[U][Q];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t co = c0 + u < chunks ? (uint32_t)(c0 + u) * (uint32_t)d * 4u : kFar;
#pragma unroll
            for (int q = 0; q < Q; ++q)
                v[u][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, base[q] + co, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                sum[4 * q] += __uint_as_float(v[u][q].x);
                sum[4 * q + 1] += __uint_as_float(v[u][q].y);
                sum[4 * q + 2] += __uint_as_float(v[u][q].z);
                sum[4 * q + 3] += __uint_as_float(v[u][q].w);
            }
    }
    float vals[E];
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        vals[e] = __fsqrt_rn(sum[e]);
        key[e] = score_key(vals[e]);
    }
    block_select<BS, E>(sh, key, nv, j0, k, idx_all ? idx_all + b * ld_idx : nullptr,
                        pad_all ? pad_all + b * ld_pad : nullptr, ld_pad, nullptr, vals, sel_out, nullptr);
}

// Final column norms: 64 columns per workgroup, 16 row-chunk groups per
// column; group g sums the chunks g, g+16, ... in ascending order (four loads
// in flight), the 16 group sums are added in a fixed tree order, then a
// correctly rounded sqrt.
__global__ __launch_bounds__(1024) void finalize_kernel(const float *__restrict__ part, int64_t chunks, int d,
                                                        float *__restrict__ s_all) {
    __shared__ float red[16][64];
    const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 64 + c;
    float *s = s_all + b * d;
    float sum = 0.f;
    if (j < d) {
        const float *p = part + b * chunks * d + j;
        int64_t r = g;
        for (; r + 48 < chunks; r += 64) {
            const float v0 = p[r * d], v1 = p[(r + 16) * d], v2 = p[(r + 32) * d], v3 = p[(r + 48) * d];
            sum += v0;
            sum += v1;
            sum += v2;
            sum += v3;
        }
        for (; r < chunks; r += 16) sum += p[r * d];
    }
    red[g][c] = sum;
    __syncthreads();
    if (g == 0 && j < d) {
        float t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = red[2 * q][c] + red[2 * q + 1][c];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = t[2 * q] + t[2 * q + 1];
        s[j] = __fsqrt_rn((t[0] + t[1]) + (t[2] + t[3]));
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
unsigned g_norm_select_attr_done = 0;

// Attention's selection and K pack in one launch.  Workgroup (x, b) of
// query head b ranks the head's D column norms itself from the row-chunk
// partials of Q: the same fp32 sum in ascending chunk order, correctly
// rounded square root and order-preserving key as norm_select_kernel, so the
// same kept set (the k largest keys, ties to the lower index, listed in
// ascending order).  It then packs K_g[:, I_b] for its 256 rows as
// pack_short_rows_kernel does, reading the kept columns from LDS.  Workgroup
// (0, b) also writes the head's kept list (idx, k entries, when given) and
// the padded list (pad, kpad entries, -1 past k) that the attention kernel
// reads.  The rows' loads are issued first, so the ranking runs while they
// are in flight.  Ranking: key t's rank is the number of keys above it plus
// the equal keys at lower indices (a strict total order, so exactly k ranks
// fall below k); its position in the list is the number of kept indices
// below t.
template <int D>
__global__ __launch_bounds__(256) void select_pack_short_kernel(const float *__restrict__ part_all, int chunks, int k,
                                                                int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                                int32_t *__restrict__ pad_all, int64_t kpad,
                                                                const uint16_t *__restrict__ src, int64_t rows,
                                                                int64_t ld_src, int64_t src_stride, int64_t group,
                                                                uint16_t *__restrict__ dst, int64_t dst_stride) {
    constexpr int CPR = D / 8;         // 16-byte chunks per row
    constexpr int STRIDE = D / 4 + 1;  // 8-byte words per LDS row (odd)
    constexpr int PER = CPR;           // chunk loads per thread
    constexpr int PF = 8;              // partials loaded ahead of the rows
    __shared__ uint2 rowl[256 * STRIDE];
    __shared__ __align__(16) uint32_t skey[D];
    __shared__ int32_t ssel[D];  // kept columns ascending, then -1 (kpad <= D)
    __shared__ int swave0;       // kept columns among the first 64
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t b = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * 256;
    const uint16_t *S = src + (b / group) * src_stride;
    uint16_t *Dp = dst + b * dst_stride;
    const int nr = (int)min((int64_t)256, rows - r0);
    const float *part = part_all + b * (int64_t)chunks * D + tid;

    // the first PF partials of column tid go out before the rows' loads, so
    // their wait does not cover the rows
    float pv[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) pv[u] = (tid < D && u < chunks) ? part[(int64_t)u * D] : 0.f;
    uint4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * 256 + tid;  // chunk e: row e / CPR, chunk e % CPR
        const int r = e / CPR, c = e % CPR;
        v[u] = r < nr ? *reinterpret_cast<const uint4 *>(S + (r0 + r) * ld_src + c * 8) : make_uint4(0, 0, 0, 0);
    }
    if (tid < D) {
        // ascending chunk order; the zeros past the last chunk leave the sum unchanged
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < PF; ++u) sum += pv[u];
        for (int c = PF; c < chunks; ++c) sum += part[(int64_t)c * D];
        skey[tid] = score_key(__fsqrt_rn(sum));
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * 256 + tid;
        const int r = e / CPR, c = e % CPR;
        rowl[r * STRIDE + 2 * c] = make_uint2(v[u].x, v[u].y);
        rowl[r * STRIDE + 2 * c + 1] = make_uint2(v[u].z, v[u].w);
    }
    __syncthreads();
    bool kept = false;
    uint64_t mask = 0;
    if (tid < D) {  // whole waves: D is 64 or 128
        const uint32_t key = skey[tid];
        int rank = 0;
        const uint4 *k4 = reinterpret_cast<const uint4 *>(skey);
#pragma unroll 8
        for (int q = 0; q < D / 4; ++q) {
            const uint4 kq = k4[q];
            const uint32_t kj[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) rank += (kj[e] > key) || (kj[e] == key && 4 * q + e < tid);
        }
        kept = rank < k;
        mask = __ballot(kept);
        if (tid == 0) swave0 = __popcll(mask);
    }
    __syncthreads();
    if (tid < D) {
        const int pos = __popcll(mask & ((1ull << lane) - 1)) + (tid >= 64 ? swave0 : 0);
        if (kept) ssel[pos] = tid;
        if (tid >= k) ssel[tid] = -1;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int t = tid; t < kpad; t += 256) {
            const int32_t j = ssel[t];
            pad_all[b * kpad + t] = j;
            if (idx_all && t < k) idx_all[b * ld_idx + t] = j;
        }
    }
    const uint16_t *mine = reinterpret_cast<const uint16_t *>(rowl + tid * STRIDE);
    const int64_t row = r0 + tid;
    const int64_t blk = row >> 5;
    if (row >= ((rows + 31) & ~(int64_t)31)) return;  // past the last 32-row block of the output
#pragma unroll 2
    for (int c = 0; c < (int)(kpad / 8); ++c) {
        int32_t j[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) j[e] = ssel[c * 8 + e];
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = mine[max(j[e], 0)];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (j[e] >= 0 && tid < nr) ? h[e] : 0u;
        *reinterpret_cast<uint4 *>(Dp + ((blk * (kpad >> 4) + (c >> 1)) * 64 + (c & 1) * 32 + (row & 31)) * 8) =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
}

}  // namespace

// Strips of 16 threads x one 16-byte load (128 bf16 / 64 fp32 columns: one
// 256-byte segment per row) and a few hundred workgroups, each thread summing
// at least 8 rows: the fastest shape measured on MI355X for the 4096 x 4096
// bf16 activation block (7.4 us, 4.6 TB/s, against 13-15 us for 512-column
// strips).
ColnormPlan colnorm_plan(rmm_dtype_t dt, int64_t n, int64_t d, int64_t batch) {
    const int V = dt == RMM_BF16 ? 8 : 4;
    ColnormPlan p;
    if (dt == RMM_BF16) {
        // 128- or 256-column strips; rows per thread 8, 16 or 32, whichever
        // first brings the grid to at most ~768 workgroups and, for d <= 4096
        // (where one workgroup per batch entry reads every partial before its
        // selection), the row chunks to at most 8: one round of loads there.
        // On the 4096 x 4096 block, 8 chunks instead of 16 cost the partial
        // pass 0.2 us and save the selection 1 us.
        int tc = d <= 4096 ? 16 : 32;
        while (tc > 1 && (int64_t)tc * V / 2 >= d) tc /= 2;
        const int tr = kNormThreads / tc;
        p.tc = tc;
        p.strips = (int)((d + (int64_t)tc * V - 1) / ((int64_t)tc * V));
        int rpt = 8;
        for (;;) {
            const int64_t chunks = (n + (int64_t)tr * rpt - 1) / ((int64_t)tr * rpt);
            if (rpt == 32 || ((int64_t)p.strips * batch * chunks <= 768 && (d > 4096 || chunks <= 8))) break;
            rpt *= 2;
        }
        p.rpt = rpt;
        p.rows_per_chunk = (int64_t)tr * rpt;
        p.chunks = (int)((n + p.rows_per_chunk - 1) / p.rows_per_chunk);
        return p;
    }
    int tc = 16;
    while (tc > 1 && (int64_t)tc * V / 2 >= d) tc /= 2;
    const int tr = kNormThreads / tc;
    p.tc = tc;
    p.rpt = 0;
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
    const int64_t a_bytes = ((n - 1) * lda + d) * 2;  // one batch entry
    if (dt == RMM_BF16 && p.rpt > 0 && vec_ok && d % 8 == 0 && a_bytes < 0x7fffffff) {
        const uint16_t *Ab = static_cast<const uint16_t *>(A);
        if (p.rpt == 8)
            colnorm_rows_kernel<8><<<grid, kNormThreads, 0, stream>>>(Ab, n, d, lda, strideA, p.tc, p.rows_per_chunk,
                                                                       a_bytes, part);
        else if (p.rpt == 16)
            colnorm_rows_kernel<16><<<grid, kNormThreads, 0, stream>>>(Ab, n, d, lda, strideA, p.tc, p.rows_per_chunk,
                                                                        a_bytes, part);
        else
            colnorm_rows_kernel<32><<<grid, kNormThreads, 0, stream>>>(Ab, n, d, lda, strideA, p.tc, p.rows_per_chunk,
                                                                        a_bytes, part);
        return hipGetLastError();
    }
    if (dt == RMM_BF16)
        colnorm_partial_kernel<uint16_t><<<grid, kNormThreads, 0, stream>>>(
            static_cast<const uint16_t *>(A), n, d, lda, strideA, p.tc, p.rows_per_chunk, vec_ok, part);
    else
        colnorm_partial_kernel<float><<<grid, kNormThreads, 0, stream>>>(
            static_cast<const float *>(A), n, d, lda, strideA, p.tc, p.rows_per_chunk, vec_ok, part);
    return hipGetLastError();
}

// Tiles of 128 columns x 128 rows (256-byte runs on both sides, 64 KB of
// LDS: two workgroups per CU).  A chunk takes 1, 2 or 4 tiles: as many as
// still give at least 256 workgroups, and more where that keeps the
// partials within what the fused norm+select kernel takes.  Measured on
// MI355X inside the product's step (2 to 8 rotated input copies): 24.9 us
// for the 2048 x 14336 block (4 tiles per chunk) and 29.5 us for 4096 x 8192
// (4), against 29.4 and 32.3 us for 64-column strips read in 128-byte runs
// with every load issued up front; 4096 x 4096 (4 tiles, 8 chunks) 18.9 us
// against 19.8.  Two tiles per chunk there (512 workgroups) took 17.5 us but
// doubles the partials, which the selection then reads in 1.1 us more.
constexpr int kTransTC = 128, kTransTR = 128, kTransThreads = 256, kTransMaxTiles = 4;
constexpr int64_t kTransMinGroups = 256;

ColnormPlan colnorm_transpose_plan(int64_t n, int64_t d) {
    ColnormPlan p;
    p.tc = 0;
    p.strips = (int)((d + kTransTC - 1) / kTransTC);
    auto groups = [&](int64_t rows) { return (int64_t)p.strips * ((n + rows - 1) / rows); };
    int64_t rows = kTransTR;
    while (rows < (int64_t)kTransTR * kTransMaxTiles && groups(2 * rows) >= kTransMinGroups) rows *= 2;
    while (rows < (int64_t)kTransTR * kTransMaxTiles && !norm_select_ok((n + rows - 1) / rows, d) &&
           norm_select_ok((n + 2 * rows - 1) / (2 * rows), d) && groups(2 * rows) >= kTransMinGroups / 2)
        rows *= 2;
    p.rows_per_chunk = rows;
    p.rpt = (int)(rows / kTransTR);
    p.chunks = (int)((n + rows - 1) / rows);
    return p;
}

hipError_t launch_colnorm_transpose(const void *A, int64_t n, int64_t d, int64_t lda, const ColnormPlan &p,
                                    uint16_t *At, int64_t ldt, float *part, hipStream_t stream) {
    const int64_t a_bytes = ((n - 1) * lda + d) * 2;
    if (n % 8 || d % 8 || lda % 8 || ldt % 8 || ((uintptr_t)A & 15) || ((uintptr_t)At & 15) ||
        a_bytes >= 0x7fffffff || p.rows_per_chunk % kTransTR || p.rows_per_chunk < kTransTR ||
        p.strips != (d + kTransTC - 1) / kTransTC)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)p.strips, (unsigned)p.chunks);
    colnorm_transpose_kernel<kTransTC, kTransTR, kTransThreads><<<grid, kTransThreads, 0, stream>>>(
        static_cast<const uint16_t *>(A), n, d, lda, p.rows_per_chunk, a_bytes, At, ldt, part);
    return hipGetLastError();
}

hipError_t launch_colnorm_finalize(const float *part, int64_t chunks, int64_t d, int64_t batch, float *s,
                                   hipStream_t stream) {
    dim3 grid((unsigned)((d + 63) / 64), (unsigned)batch);
    finalize_kernel<<<grid, 1024, 0, stream>>>(part, chunks, (int)d, s);
    return hipGetLastError();
}

hipError_t launch_norm_select(const float *part, int64_t chunks, int64_t d, int64_t batch, int64_t k, int32_t *idx,
                              int64_t ld_idx, int32_t *idx_pad, int64_t ld_pad, hipStream_t stream) {
    if (!norm_select_ok(chunks, d) || ((uintptr_t)part & 15)) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (dev < 32 && !(g_norm_select_attr_done & (1u << dev))) {
        const void *fns[3] = {reinterpret_cast<const void *>(&norm_select_kernel<4>),
                              reinterpret_cast<const void *>(&norm_select_kernel<8>),
                              reinterpret_cast<const void *>(&norm_select_kernel<16>)};
        for (const void *f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
            if (e != hipSuccess) return e;
        }
        g_norm_select_attr_done |= 1u << dev;
    }
    // E keys per thread: 1024 threads cover d
    const size_t lds = (size_t)k * 4;
    if (d <= 4096)
        norm_select_kernel<4><<<(unsigned)batch, 1024, lds, stream>>>(part, (int)chunks, (int)d, (int)k, idx, ld_idx,
                                                                      idx_pad, ld_pad);
    else if (d <= 8192)
        norm_select_kernel<8><<<(unsigned)batch, 1024, lds, stream>>>(part, (int)chunks, (int)d, (int)k, idx, ld_idx,
                                                                      idx_pad, ld_pad);
    else
        norm_select_kernel<16><<<(unsigned)batch, 1024, lds, stream>>>(part, (int)chunks, (int)d, (int)k, idx, ld_idx,
                                                                       idx_pad, ld_pad);
    return hipGetLastError();
}

// Scores are staged in LDS when they fit comfortably (d <= 24576 keys, 96 KB).
static constexpr int64_t kSelectLdsKeys = 24576;

hipError_t launch_select(const float *s, const void *a_src, rmm_dtype_t a_dt, int64_t a_stride, int64_t batch,
                         int64_t d, int64_t k, int32_t *idx, int64_t ld_idx, int32_t *idx_pad, int64_t ld_pad,
                         float *aval, hipStream_t stream) {
    const int a_bf16 = a_dt == RMM_BF16;
    const unsigned g = (unsigned)batch;
    // dynamic LDS for the staged outputs (<= 128 KB: d <= 16384)
    const size_t out_lds = (size_t)k * 4 * (aval ? 2 : 1);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (dev < 32 && !(g_select_attr_done & (1u << dev))) {
        const void *ks[] = {reinterpret_cast<const void *>(&select_kernel<1024, 16, true, true>),
                            reinterpret_cast<const void *>(&select_kernel<1024, 16, false, true>),
                            reinterpret_cast<const void *>(&select_kernel<1024, 16, false, false>),
                            reinterpret_cast<const void *>(&select_kernel<1024, 8, true, true>),
                            reinterpret_cast<const void *>(&select_kernel<1024, 8, false, true>),
                            reinterpret_cast<const void *>(&select_kernel<1024, 8, false, false>),
                            reinterpret_cast<const void *>(&select_big_kernel<1024>)};
        for (const void *kf : ks) {
            hipError_t e = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
            if (e != hipSuccess) return e;
        }
        g_select_attr_done |= 1u << dev;
    }
    if (a_src && a_dt == RMM_BF16) {
        if ((uintptr_t)a_src % 16 != 0 || a_stride % 8 != 0 || d > 16384) return hipErrorInvalidValue;
        const void *src = a_src;
        if (d <= 256)
            select_kernel<64, 8, true, true><<<g, 64, out_lds, stream>>>(src, a_stride, (int)d, (int)k, idx, ld_idx,
                                                                          idx_pad, ld_pad, aval);
        else if (d <= 4096)
            select_kernel<256, 16, true, true><<<g, 256, out_lds, stream>>>(src, a_stride, (int)d, (int)k, idx, ld_idx,
                                                                            idx_pad, ld_pad, aval);
        else if (d <= 8192)
            select_kernel<1024, 8, true, true><<<g, 1024, out_lds, stream>>>(src, a_stride, (int)d, (int)k, idx,
                                                                             ld_idx, idx_pad, ld_pad, aval);
        else
            select_kernel<1024, 16, true, true><<<g, 1024, out_lds, stream>>>(src, a_stride, (int)d, (int)k, idx,
                                                                              ld_idx, idx_pad, ld_pad, aval);
        return hipGetLastError();
    }
    const bool vec = ((uintptr_t)s % 16 == 0) && (d % 4 == 0);
    if (d <= 256) {
        if (vec)
            select_kernel<64, 4, false, true><<<g, 64, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx, idx_pad,
                                                                           ld_pad, aval);
        else
            select_kernel<64, 4, false, false><<<g, 64, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx, idx_pad,
                                                                            ld_pad, aval);
    } else if (d <= 4096) {
        if (vec)
            select_kernel<256, 16, false, true><<<g, 256, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx,
                                                                             idx_pad, ld_pad, aval);
        else
            select_kernel<256, 16, false, false><<<g, 256, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx,
                                                                              idx_pad, ld_pad, aval);
    } else if (d <= 8192) {
        if (vec)
            select_kernel<1024, 8, false, true><<<g, 1024, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx,
                                                                              idx_pad, ld_pad, aval);
        else
            select_kernel<1024, 8, false, false><<<g, 1024, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx,
                                                                               idx_pad, ld_pad, aval);
    } else if (d <= 16384) {
        if (vec)
            select_kernel<1024, 16, false, true><<<g, 1024, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx,
                                                                               idx_pad, ld_pad, aval);
        else
            select_kernel<1024, 16, false, false><<<g, 1024, out_lds, stream>>>(s, d, (int)d, (int)k, idx, ld_idx,
                                                                                idx_pad, ld_pad, aval);
    } else {
        const int use_lds = d <= kSelectLdsKeys;
        const size_t lds = use_lds ? (size_t)d * 4 : 0;
        select_big_kernel<1024><<<g, 1024, lds, stream>>>(s, a_src, a_bf16, a_stride, d, k, idx, ld_idx, idx_pad,
                                                          ld_pad, aval, use_lds);
    }
    return hipGetLastError();
}

hipError_t launch_index_prepare(const int32_t *idx, int64_t batch, int64_t k, int64_t d, int32_t *idx_pad,
                                int64_t ld_pad, const void *a_row, float *aval, hipStream_t stream) {
    if (k < 1 || ld_pad < k || batch < 1 || batch > 65535 || d > INT32_MAX || (aval && (!a_row || batch != 1)))
        return hipErrorInvalidValue;
    index_prepare_kernel<1024, 4><<<(unsigned)batch, 1024, 0, stream>>>(idx, k, d, idx_pad, ld_pad,
                                                                        static_cast<const uint16_t *>(a_row), aval);
    return hipGetLastError();
}

hipError_t launch_iota(int32_t *idx, int64_t k, int64_t ld, int64_t batch, hipStream_t stream) {
    int64_t total = ld * batch;
    iota_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(idx, k, ld, total);
    return hipGetLastError();
}

bool select_pack_short_ok(int64_t d, int64_t k, int64_t kpad, int64_t chunks) {
    return (d == 64 || d == 128) && k >= 1 && k <= d && kpad % 64 == 0 && kpad >= k && kpad <= d && chunks >= 1 &&
           chunks <= kSelectPackMaxChunks;
}

hipError_t launch_select_pack_short(const float *part, int64_t chunks, int64_t k, int32_t *idx, int64_t ld_idx,
                                    int32_t *pad, int64_t kpad, const void *src, int64_t rows, int64_t d,
                                    int64_t ld_src, int64_t src_stride, int64_t group, void *dst, int64_t dst_stride,
                                    int64_t batch, hipStream_t stream) {
    if (!select_pack_short_ok(d, k, kpad, chunks) || !part || !pad || !src || !dst || rows < 1 || group < 1 ||
        batch < 1 || batch > 65535 || (uintptr_t)src % 16 || ld_src % 8 || src_stride % 8 || (uintptr_t)dst % 16 ||
        (rows + 255) / 256 > INT32_MAX)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)((rows + 255) / 256), (unsigned)batch);
    const uint16_t *sp = static_cast<const uint16_t *>(src);
    uint16_t *dp = static_cast<uint16_t *>(dst);
    if (d == 64)
        select_pack_short_kernel<64><<<grid, 256, 0, stream>>>(part, (int)chunks, (int)k, idx, ld_idx, pad, kpad, sp,
                                                               rows, ld_src, src_stride, group, dp, dst_stride);
    else
        select_pack_short_kernel<128><<<grid, 256, 0, stream>>>(part, (int)chunks, (int)k, idx, ld_idx, pad, kpad, sp,
                                                                rows, ld_src, src_stride, group, dp, dst_stride);
    return hipGetLastError();
}

}  // namespace rmm
