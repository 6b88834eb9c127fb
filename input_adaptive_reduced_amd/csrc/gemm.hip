// Gather and reduced-product kernels for gfx950.
//
// Steps 3 and 4 of reduced matrix multiplication ("Reduced Matrix
// Multiplication: Input-Adaptive Matrix-Product Reduction for LLM Inference",
// Sec. 3.2 and eqs. (3)-(4) of App. D.1): once the kept index set I is known,
// compute only A[:, I] B[I, :], cutting the contraction from d to
// k = ceil(rho d).  The product is a dense contraction over k, so it runs on
// the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Operand handling
//  * A's kept columns are strided 2-byte elements of row-major A, so they are
//    first packed into a k-contiguous buffer (pack_kernel: each workgroup
//    stages whole rows of A in LDS with 16-byte loads and gathers from LDS),
//    padded with zeros to a multiple of the 64-wide K step.
//  * B's kept rows are contiguous.  With B stored d x m the GEMM reads them in
//    place through the index list (bmode 0): each thread fetches an 8 x 8
//    block (8 gathered rows x 8 columns, 16-byte loads), transposes it in
//    registers and writes eight k-contiguous 16-byte vectors to LDS, the
//    layout the MFMA B operand wants.  With B stored as B^T (m x d: the keys
//    of Q K^T) the kept columns are packed like A (bmode 1).
//  * LDS tiles hold rows of 64 bf16 (eight 16-byte chunks); chunk c of row r
//    lives at c ^ ((r ^ (r >> 3)) & 7), which keeps both the transposed
//    stores (rows 8 apart) and the MFMA operand reads (consecutive rows)
//    free of bank conflicts.
//  * Tiles are 256x256 (4 waves, 128x128 each) or 128x128, double-buffered in
//    LDS; workgroup ids are remapped so that each XCD (ids are dealt to the 8
//    XCDs round-robin) works on a compact block of output tiles and shares
//    its A rows and B columns in its own L2.
//  * Shapes with too few tiles to fill 256 CUs split the K range; fp32
//    partials are then added in split order by splitk_reduce (deterministic).
#include "rmm_internal.h"

namespace rmm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int BK = 64;  // K step: 64 bf16 = eight 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    union {
        uint4 u;
        bf16x8_t b;
    } x;
    x.u = v;
    return x.b;
}

// 8x8 transpose of 2-byte elements: in[r] holds row r (8 columns); out[c]
// receives column c (8 rows).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint4 &x = in[2 * p];
            const uint4 &y = in[2 * p + 1];
            uint32_t xd = (c >> 1) == 0 ? x.x : (c >> 1) == 1 ? x.y : (c >> 1) == 2 ? x.z : x.w;
            uint32_t yd = (c >> 1) == 0 ? y.x : (c >> 1) == 1 ? y.y : (c >> 1) == 2 ? y.z : y.w;
            w[p] = (c & 1) ? ((xd >> 16) | (yd & 0xffff0000u)) : ((xd & 0xffffu) | (yd << 16));
        }
        out[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Tile index -> (tm, tn): XCD-compact, then grouped by GM tile rows.
__device__ __forceinline__ void tile_coords(int t, int T, int tiles_m, int tiles_n, int &tm, int &tn) {
    if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
    constexpr int GM = 4;
    const int per_group = GM * tiles_n;
    const int g = t / per_group;
    const int first = g * GM;
    const int gsz = min(GM, tiles_m - first);
    const int in = t - g * per_group;
    tm = first + in % gsz;
    tn = in / gsz;
}

template <int BM, int BN, int WM, int WN, int BMODE, bool SPLIT>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_PER = BM * 8 / NT;
    constexpr int B_PER = BN * 8 / NT;  // bmode 1
    static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
    static_assert(BMODE == 1 || BN <= NT, "bmode 0 needs one 8x8 B block per thread at most");

    __shared__ uint4 sA[2][BM * 8];
    __shared__ uint4 sB[2][BN * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const int tiles_m = (int)((g.n + BM - 1) / BM);
    const int tiles_n = (int)((g.m + BN - 1) / BN);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t b = blockIdx.z;
    const int split = blockIdx.y;

    const uint16_t *A = g.A + b * g.strideA;
    const uint16_t *B = g.B + (b / g.group) * g.strideB;
    const int32_t *idx = g.idx ? g.idx + b * g.ld_idx : nullptr;

    const int KT = (int)(g.kpad / BK);
    const int per = (KT + g.splits - 1) / g.splits;
    const int kt0 = split * per;
    const int kt1 = min(KT, kt0 + per);

    uint4 ra[A_PER];
    uint4 rb[BMODE == 0 ? 8 : B_PER];

    auto load_a = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int c = tid + i * NT;
            const int r = c >> 3, ch = c & 7;
            const int64_t gr = m0 + r;
            ra[i] = gr < g.n ? *reinterpret_cast<const uint4 *>(A + gr * g.lda + (int64_t)kt * BK + ch * 8)
                             : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int c = tid + i * NT;
            const int r = c >> 3, ch = c & 7;
            sA[buf][r * 8 + swz(r, ch)] = ra[i];
        }
    };
    auto load_b = [&](int kt) {
        if constexpr (BMODE == 0) {
            if (tid < BN) {
                const int kq = tid / (BN / 8), nc = tid % (BN / 8);
                const int64_t col = n0 + nc * 8;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int64_t t = (int64_t)kt * BK + kq * 8 + r;
                    const int64_t gi = t < g.k ? (idx ? (int64_t)idx[t] : t) : -1;
                    rb[r] = (gi >= 0 && col < g.m) ? *reinterpret_cast<const uint4 *>(B + gi * g.ldb + col)
                                                   : make_uint4(0, 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int c = tid + i * NT;
                const int r = c >> 3, ch = c & 7;
                const int64_t gr = n0 + r;
                rb[i] = gr < g.m ? *reinterpret_cast<const uint4 *>(B + gr * g.ldb + (int64_t)kt * BK + ch * 8)
                                 : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_b = [&](int buf) {
        if constexpr (BMODE == 0) {
            if (tid < BN) {
                const int kq = tid / (BN / 8), nc = tid % (BN / 8);
                uint4 ob[8];
                transpose8x8(rb, ob);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int nn = nc * 8 + c;
                    sB[buf][nn * 8 + swz(nn, kq)] = ob[c];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_PER; ++i) {
                const int c = tid + i * NT;
                const int r = c >> 3, ch = c & 7;
                sB[buf][r * 8 + swz(r, ch)] = rb[i];
            }
        }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    if (kt0 < kt1) {
        load_a(kt0);
        load_b(kt0);
        store_a(0);
        store_b(0);
        __syncthreads();
        for (int kt = kt0; kt < kt1; ++kt) {
            const int cur = (kt - kt0) & 1;
            const bool more = kt + 1 < kt1;
            if (more) {
                load_a(kt + 1);
                load_b(kt + 1);
            }
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int ch = ks * 2 + (lane >> 5);
                bf16x8_t fa[FM], fb[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wm * WTM + i * 32 + (lane & 31);
                    fa[i] = as_bf16x8(sA[cur][r * 8 + swz(r, ch)]);
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int nn = wn * WTN + j * 32 + (lane & 31);
                    fb[j] = as_bf16x8(sB[cur][nn * 8 + swz(nn, ch)]);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
            if (more) {
                store_a(cur ^ 1);
                store_b(cur ^ 1);
            }
            __syncthreads();
        }
    }

    // epilogue: lane l, register e of a 32x32 block holds row
    // (e/4)*8 + (l/32)*4 + e%4 and column l%32.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = n0 + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * WTM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                if (row < g.n && col < g.m) {
                    if constexpr (SPLIT) {
                        g.part[(((int64_t)split * g.batch + b) * g.n + row) * g.m + col] = acc[i][j][e];
                    } else {
                        g.Y[b * g.strideY + row * g.ldy + col] = f32_to_bf16(g.alpha * acc[i][j][e]);
                    }
                }
            }
        }
    }
}

// Y = alpha * sum over splits (ascending) of the fp32 partials; 4 columns per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int splits, int64_t n,
                                                            int64_t m, int64_t batch, float alpha,
                                                            uint16_t *__restrict__ Y, int64_t ldy, int64_t strideY) {
    const int64_t q = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t plane = n * m;
    const int64_t total = plane * batch;
    if (q >= total) return;
    const int64_t b = q / plane;
    const int64_t rc = q - b * plane;
    const int64_t row = rc / m, col = rc - row * m;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < splits; ++sp) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)sp * total + q);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    uint16_t *y = Y + b * strideY + row * ldy + col;
    uint32_t lo = uint32_t(f32_to_bf16(alpha * s.x)) | (uint32_t(f32_to_bf16(alpha * s.y)) << 16);
    uint32_t hi = uint32_t(f32_to_bf16(alpha * s.z)) | (uint32_t(f32_to_bf16(alpha * s.w)) << 16);
    *reinterpret_cast<uint2 *>(y) = make_uint2(lo, hi);
}

// ------------------------------------------------------------------ pack
// dst[b][r][t] = src[b/group][r][idx[b][t]] (t < k), 0 for k <= t < kpad.
// Whole source rows are staged in LDS (16-byte loads when aligned) when
// `rows_per_wg` rows of d elements fit; otherwise gathers go to global memory.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ src, int64_t rows, int64_t d,
                                                   int64_t ld_src, int64_t src_stride, int64_t group,
                                                   const int32_t *__restrict__ idx_all, int64_t ld_idx, int64_t k,
                                                   int64_t kpad, uint16_t *__restrict__ dst, int64_t dst_stride,
                                                   int rows_per_wg, int use_lds, int vec_ok) {
    extern __shared__ uint16_t rowbuf[];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nr = (int)min((int64_t)rows_per_wg, rows - r0);
    const uint16_t *S = src + (b / group) * src_stride;
    const int32_t *idx = idx_all + b * ld_idx;
    uint16_t *D = dst + b * dst_stride;

    if (use_lds) {
        if (vec_ok) {
            const int64_t vpr = d / 8;  // d % 8 == 0 when vec_ok
            for (int64_t q = tid; q < (int64_t)nr * vpr; q += 256) {
                const int64_t rr = q / vpr, c = q - rr * vpr;
                reinterpret_cast<uint4 *>(rowbuf + rr * d)[c] =
                    *reinterpret_cast<const uint4 *>(S + (r0 + rr) * ld_src + c * 8);
            }
        } else {
            for (int64_t q = tid; q < (int64_t)nr * d; q += 256) {
                const int64_t rr = q / d, c = q - rr * d;
                rowbuf[q] = S[(r0 + rr) * ld_src + c];
            }
        }
        __syncthreads();
    }
    const int64_t cpr = kpad / 8;  // output chunks per row
    for (int64_t q = tid; q < (int64_t)nr * cpr; q += 256) {
        const int64_t rr = q / cpr, c = q - rr * cpr;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t h[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int64_t t = c * 8 + 2 * p + e;
                uint16_t v = 0;
                if (t < k) {
                    const int64_t j = idx[t];
                    v = use_lds ? rowbuf[rr * d + j] : S[(r0 + rr) * ld_src + j];
                }
                h[e] = v;
            }
            w[p] = h[0] | (h[1] << 16);
        }
        *reinterpret_cast<uint4 *>(D + (r0 + rr) * kpad + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ------------------------------------------------------------------ generic SIMT path
template <typename T>
struct Elem;
template <>
struct Elem<float> {
    __device__ static float ld(const float *p) { return *p; }
    __device__ static void st(float *p, float v) { *p = v; }
};
template <>
struct Elem<uint16_t> {
    __device__ static float ld(const uint16_t *p) { return bf16_to_f32(*p); }
    __device__ static void st(uint16_t *p, float v) { *p = f32_to_bf16(v); }
};

// 64x64 output tile per 256 threads, 4x4 outputs per thread, K chunks of 16
// gathered through the index list; fp32 FMA in ascending t.
template <typename T>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GenericArgs g) {
    __shared__ float sA[16][64 + 1];
    __shared__ float sB[16][64 + 1];
    __shared__ int32_t sIdx[16];
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int64_t b = blockIdx.z;
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const T *A = static_cast<const T *>(g.A) + b * g.strideA;
    const T *B = static_cast<const T *>(g.B) + (b / g.group) * g.strideB;
    const int32_t *idx = g.idx ? g.idx + b * g.ld_idx : nullptr;
    T *Y = static_cast<T *>(g.Y) + b * g.strideY;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int64_t t0 = 0; t0 < g.k; t0 += 16) {
        if (threadIdx.x < 16) {
            const int64_t t = t0 + threadIdx.x;
            sIdx[threadIdx.x] = t < g.k ? (idx ? idx[t] : (int32_t)t) : -1;
        }
        __syncthreads();
        for (int q = threadIdx.x; q < 16 * 64; q += 256) {
            const int kk = q / 64, c = q % 64;
            const int32_t j = sIdx[kk];
            const int64_t row = m0 + c;
            sA[kk][c] = (j >= 0 && row < g.n) ? Elem<T>::ld(A + row * g.lda + j) : 0.f;
            const int64_t col = n0 + c;
            float bv = 0.f;
            if (j >= 0 && col < g.m) bv = g.transB ? Elem<T>::ld(B + col * g.ldb + j) : Elem<T>::ld(B + (int64_t)j * g.ldb + col);
            sB[kk][c] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = sB[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + ty + 16 * i;
        if (row >= g.n) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + tx + 16 * j;
            if (col < g.m) Elem<T>::st(Y + row * g.ldy + col, g.alpha * acc[i][j]);
        }
    }
}

unsigned g_pack_attr_done = 0;  // bit per device

template <typename K>
hipError_t allow_big_lds(K kernel) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               160 * 1024 - 1024);
}

}  // namespace

GemmConfig gemm_choose(int64_t n, int64_t m, int64_t k, int64_t batch) {
    GemmConfig c;
    const int64_t big = ((n + 255) / 256) * ((m + 255) / 256) * batch;
    const int64_t ksteps = (k + BK - 1) / BK;
    if (big >= 192) {
        c.tile = 0;
        c.splits = 1;
        return c;
    }
    const int64_t small = ((n + 127) / 128) * ((m + 127) / 128) * batch;
    if (big >= 64 && ksteps >= 32) {
        // large K: keep 256x256 tiles and split K to fill the chip
        int64_t s = (256 + big - 1) / big;
        if (s > ksteps / 16) s = ksteps / 16;
        c.tile = 0;
        c.splits = (int)(s < 1 ? 1 : s);
        return c;
    }
    c.tile = 1;
    int64_t s = small >= 256 ? 1 : (256 + small - 1) / small;
    if (s > ksteps / 8) s = ksteps / 8;
    c.splits = (int)(s < 1 ? 1 : s);
    return c;
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_tile(const GemmArgs &g, hipStream_t stream) {
    const int64_t tiles = ((g.n + BM - 1) / BM) * ((g.m + BN - 1) / BN);
    dim3 grid((unsigned)tiles, (unsigned)g.splits, (unsigned)g.batch);
    dim3 block(WM * WN * 64);
    const bool split = g.splits > 1;
    if (g.bmode == 0) {
        if (split)
            gemm_bf16_kernel<BM, BN, WM, WN, 0, true><<<grid, block, 0, stream>>>(g);
        else
            gemm_bf16_kernel<BM, BN, WM, WN, 0, false><<<grid, block, 0, stream>>>(g);
    } else {
        if (split)
            gemm_bf16_kernel<BM, BN, WM, WN, 1, true><<<grid, block, 0, stream>>>(g);
        else
            gemm_bf16_kernel<BM, BN, WM, WN, 1, false><<<grid, block, 0, stream>>>(g);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs &g, const GemmConfig &c, hipStream_t stream) {
    GemmArgs a = g;
    a.splits = c.splits;
    if (c.tile == 0) return launch_tile<256, 256, 2, 2>(a, stream);
    return launch_tile<128, 128, 2, 2>(a, stream);
}

hipError_t launch_splitk_reduce(const float *part, int splits, int64_t n, int64_t m, int64_t batch, float alpha,
                                uint16_t *Y, int64_t ldy, int64_t strideY, hipStream_t stream) {
    const int64_t quads = n * m * batch / 4;
    splitk_reduce_kernel<<<(unsigned)((quads + 255) / 256), 256, 0, stream>>>(part, splits, n, m, batch, alpha, Y,
                                                                            ldy, strideY);
    return hipGetLastError();
}

// LDS budget for staged rows in pack_kernel.
static constexpr int64_t kPackLdsBytes = 64 * 1024;

hipError_t launch_pack(const void *src, rmm_dtype_t dt, int64_t rows, int64_t d, int64_t ld_src, int64_t src_stride,
                       int64_t group, const int32_t *idx, int64_t ld_idx, int64_t k, int64_t kpad, void *dst,
                       int64_t dst_stride, int64_t batch, hipStream_t stream) {
    if (dt != RMM_BF16) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (dev < 32 && !(g_pack_attr_done & (1u << dev))) {
        hipError_t e = allow_big_lds(&pack_kernel);
        if (e != hipSuccess) return e;
        g_pack_attr_done |= 1u << dev;
    }
    const int64_t row_bytes = d * 2;
    int rpw = (int)(kPackLdsBytes / row_bytes);
    int use_lds = rpw >= 1;
    if (rpw > 8) rpw = 8;
    if (rpw < 1) rpw = 4;
    const int vec_ok = use_lds && ((uintptr_t)src % 16 == 0) && (ld_src % 8 == 0) && (d % 8 == 0) &&
                       (src_stride % 8 == 0);
    const size_t lds = use_lds ? (size_t)rpw * (size_t)row_bytes : 0;
    dim3 grid((unsigned)((rows + rpw - 1) / rpw), (unsigned)batch);
    pack_kernel<<<grid, 256, lds, stream>>>(static_cast<const uint16_t *>(src), rows, d, ld_src, src_stride, group,
                                            idx, ld_idx, k, kpad, static_cast<uint16_t *>(dst), dst_stride, rpw,
                                            use_lds, vec_ok);
    return hipGetLastError();
}

hipError_t launch_gemm_generic(const GenericArgs &g, hipStream_t stream) {
    dim3 grid((unsigned)((g.m + 63) / 64), (unsigned)((g.n + 63) / 64), (unsigned)g.batch);
    if (g.dt == RMM_F32)
        gemm_generic_kernel<float><<<grid, 256, 0, stream>>>(g);
    else
        gemm_generic_kernel<uint16_t><<<grid, 256, 0, stream>>>(g);
    return hipGetLastError();
}

}  // namespace rmm
