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
//    first packed (pack_blocks_kernel) into MFMA operand blocks: for 32 rows
//    and 16 kept entries, a 1 KB block in the order the lanes of one
//    32x32x16 MFMA want it, padded with zeros to whole blocks.  The main
//    kernel (gemm_adirect_kernel) then loads every A fragment straight from
//    memory into registers with one coalesced 16-byte load per lane, two K
//    steps ahead; A never passes through LDS.
//  * B's kept rows are contiguous.  With B stored d x m the kernels read them
//    in place through the index list: each thread fetches 16-byte pieces of
//    eight kept rows, stores them into a row-major LDS tile and the waves read
//    their MFMA operands with ds_read_b64_tr_b16.  With B stored as B^T
//    (m x d: the keys of Q K^T) the kept columns are packed into rows of kpad
//    entries (pack_kernel) and staged like a k-contiguous operand (bmode 1 of
//    gemm_bf16_kernel, which also serves the 128x128 tiles of small shapes).
//  * Tiles are 256x256 (4 waves, 128x128 each) or 128x128; workgroup ids are
//    remapped so that each XCD (ids are dealt to the 8 XCDs round-robin) works
//    on a compact block of output tiles and shares its A rows and B columns in
//    its own L2.
//  * Shapes with too few tiles to fill 256 CUs split the K range; fp32
//    partials are then added in split order by splitk_reduce (deterministic).
#include "rmm_internal.h"

#include <algorithm>
#include <type_traits>

namespace rmm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int BK = 64;  // K step: 64 bf16 = eight 16-byte chunks per LDS row
constexpr int kBdmaListRows = 16384;  // u16 list entries gemm_bdma_kernel keeps in LDS
constexpr int kTdmaListRows = 8192;   // u16 list entries gemm_tdma_kernel keeps in LDS
constexpr int kTdmaListRowsQ = 32768; // the same with 8-bit B (its stages take half the LDS)

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    union {
        uint4 u;
        bf16x8_t b;
    } x;
    x.u = v;
    return x.b;
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

// Buffer resource for raw buffer loads on gfx9-family parts (gfx950): loads
// at byte offsets at or beyond `bytes` return zero.  Offsets of rows that
// must read as zero (rows past n, padding entries of the index list) are
// pushed to kOob, which stays out of range while K steps are added.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int32_t nrec = (int32_t)min(bytes, (int64_t)0x7fffffff);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nrec, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}


typedef short v4i16_t __attribute__((ext_vector_type(4)));

// One workgroup computes a BM x BN output tile over a range of 64-wide K
// steps (an even number of them).  Pipeline per step kt, with two LDS
// buffers and two register staging sets:
//   * issue the global (buffer) loads of tile kt+2 into staging set kt&1
//     (gathered B rows are addressed by the index chunk loaded two steps
//     earlier) and the index chunk of tile kt+4;
//   * four k16 sub-steps of 16 MFMAs each on LDS buffer kt&1, the fragment
//     reads of the next sub-step interleaved with the current MFMAs;
//   * during sub-step 1, write staging set (kt+1)&1 (tile kt+1, loaded a
//     full step earlier) into the other LDS buffer;
//   * barrier after sub-step 2, so sub-step 3 can already read the first
//     fragments of the next buffer.
// LDS layouts: A (and packed B^T) rows of 64 bf16 in eight 16-byte chunks,
// chunk c of row r at c ^ ((r ^ r>>3) & 7); gathered B rows stay row-major
// (k rows of BN columns), chunk c of row k at c ^ 2(k & 3), and its MFMA
// operand is read with ds_read_b64_tr_b16 (lane i of a 16-lane group reads 4
// columns of row k0 + i/4; lane j receives 4 consecutive k of column j).
// Both layouts keep reads and writes free of bank conflicts.
template <int BM, int BN, int WM, int WN, int BMODE, bool SPLIT>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_PER = BM * 8 / NT;   // A chunks per thread per step
    constexpr int B_PER = BMODE == 0 ? 8 : BN * 8 / NT;
    constexpr int CPR = BN / 8;          // 16-byte chunks per row-major B row
    constexpr int B_READS = BMODE == 0 ? 2 * FN : FN;
    static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
    static_assert(BMODE == 1 || BN * 8 == NT * 8 || BN < NT, "bmode 0: one 8-row B block per thread");

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

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + b * g.strideA, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (b / g.group) * g.strideB, g.b_bytes);
    const int32_t *idx = BMODE == 0 ? g.idx + b * g.ld_idx : nullptr;

    // K steps of this split: an even count (kpad is a multiple of 128 and
    // the per-split share is rounded up to even).
    const int KT = (int)(g.kpad / BK);
    const int per = ((KT + g.splits - 1) / g.splits + 1) & ~1;
    const int kt0 = split * per;
    const int kt1 = min(KT, kt0 + per);

    // A (and bmode-1 B) staging: chunk c = tid + i*NT is tile row c/8, logical
    // 16-byte chunk c%8; rows past n (or m) read as zero.
    uint32_t aoff[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int c = tid + i * NT;
        const int64_t gr = m0 + (c >> 3);
        aoff[i] = gr < g.n ? (uint32_t)((gr * g.lda + (c & 7) * 8) * 2) : kOob;
    }
    uint32_t boff[BMODE == 1 ? B_PER : 1];
    if constexpr (BMODE == 1) {
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int c = tid + i * NT;
            const int64_t gr = n0 + (c >> 3);
            boff[i] = gr < g.m ? (uint32_t)((gr * g.ldb + (c & 7) * 8) * 2) : kOob;
        }
    }
    // bmode 0: thread owns 8 consecutive B rows (kq*8..) of one 16-byte column chunk nc
    const bool bthr = BMODE == 0 && (BN * 8 >= NT * 8 ? true : tid < BN);
    const int kq = tid / CPR, nc = tid % CPR;
    const int64_t bcol = n0 + nc * 8;

    uint4 ra0[A_PER], ra1[A_PER], rb0[B_PER], rb1[B_PER];
    int32_t ix0[8], ix1[8];

    auto load_idx = [&](int kt, int32_t (&o)[8]) {
        if constexpr (BMODE == 0) {
            if (!bthr) return;
            const int t0 = min(kt, KT - 1) * BK + kq * 8;
            const int4 p0 = *reinterpret_cast<const int4 *>(idx + t0);
            const int4 p1 = *reinterpret_cast<const int4 *>(idx + t0 + 4);
            o[0] = p0.x; o[1] = p0.y; o[2] = p0.z; o[3] = p0.w;
            o[4] = p1.x; o[5] = p1.y; o[6] = p1.z; o[7] = p1.w;
        }
    };
    auto load_tile = [&](int kt, uint4 (&ra)[A_PER], uint4 (&rb)[B_PER], const int32_t (&ix)[8]) {
        const uint32_t ko = (uint32_t)min(kt, kt1 - 1) * (BK * 2);
#pragma unroll
        for (int i = 0; i < A_PER; ++i) ra[i] = buf_load16(rA, aoff[i] + ko);
        if constexpr (BMODE == 0) {
            if (bthr) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint32_t off = ix[r] >= 0 ? (uint32_t)(((int64_t)ix[r] * g.ldb + bcol) * 2) : kOob;
                    rb[r] = buf_load16(rB, off);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_PER; ++i) rb[i] = buf_load16(rB, boff[i] + ko);
        }
    };
    auto store_tile = [&](int buf, const uint4 (&ra)[A_PER], const uint4 (&rb)[B_PER]) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int c = tid + i * NT;
            const int r = c >> 3, ch = c & 7;
            sA[buf][r * 8 + swz(r, ch)] = ra[i];
        }
        if constexpr (BMODE == 0) {
            if (bthr) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int k = kq * 8 + r;
                    sB[buf][k * CPR + (nc ^ ((k & 3) << 1))] = rb[r];
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

    auto read_frags = [&](int buf, int ks, bf16x8_t (&fa)[FM], bf16x8_t (&fb)[FN]) {
        const int ch = ks * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
            fa[i] = as_bf16x8(sA[buf][r * 8 + swz(r, ch)]);
        }
        if constexpr (BMODE == 0) {
            const int gq = lane >> 4, li = lane & 15;
            const int kbase = ks * 16 + 8 * (gq >> 1) + (li >> 2);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nn = wn * WTN + j * 32 + 16 * (gq & 1) + 4 * (li & 3);
                union {
                    v4i16_t h[2];
                    bf16x8_t v;
                } u;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = kbase + 4 * hh;
                    const char *p = reinterpret_cast<const char *>(&sB[buf][k * CPR + ((nn >> 3) ^ ((k & 3) << 1))]) +
                                    ((nn >> 2) & 1) * 8;
                    u.h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)p);
                }
                fb[j] = u.v;
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nn = wn * WTN + j * 32 + (lane & 31);
                fb[j] = as_bf16x8(sB[buf][nn * 8 + swz(nn, ch)]);
            }
        }
    };

    bf16x8_t fa[2][FM], fb[2][FN];
    auto step = [&](int kt, int buf, uint4 (&la)[A_PER], uint4 (&lb)[B_PER], int32_t (&lix)[8],
                    const uint4 (&sa)[A_PER], const uint4 (&sb)[B_PER]) {
        load_tile(kt + 2, la, lb, lix);
        load_idx(kt + 4, lix);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            if (ks + 1 < BK / 16) read_frags(buf, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            else read_frags(buf ^ 1, 0, fa[0], fb[0]);
            if (ks == 1) store_tile(buf ^ 1, sa, sb);
            // operands swapped: each lane ends up holding four consecutive
            // output columns of one output row
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
            // spread the fragment reads over the MFMAs of this sub-step
#pragma unroll
            for (int q = 0; q < FM + B_READS; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, FM * FN >= 2 * (FM + B_READS) ? 2 : 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 2) __syncthreads();
        }
    };

    if (kt0 < kt1) {
        load_idx(kt0, ix0);
        load_idx(kt0 + 1, ix1);
        load_tile(kt0, ra0, rb0, ix0);
        load_tile(kt0 + 1, ra1, rb1, ix1);
        load_idx(kt0 + 2, ix0);
        load_idx(kt0 + 3, ix1);
        store_tile(0, ra0, rb0);
        __syncthreads();
        read_frags(0, 0, fa[0], fb[0]);
        for (int kt = kt0; kt < kt1; kt += 2) {
            step(kt, 0, ra0, rb0, ix0, ra1, rb1);      // tile kt on buffer 0; tile kt+1 -> buffer 1
            step(kt + 1, 1, ra1, rb1, ix1, ra0, rb0);  // tile kt+1 on buffer 1; tile kt+2 -> buffer 0
        }
    }

    // epilogue: lane l, registers 4q..4q+3 of block (i, j) hold output row
    // i*32 + l%32 and columns j*32 + 8q + 4(l/32) + 0..3.
    if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t row = m0 + wm * WTM + i * 32 + (lane & 31);
            if (row >= g.n) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
                    if (col >= g.m) continue;  // m % 8 == 0: the four columns are all in or all out
                    *reinterpret_cast<float4 *>(g.part + (((int64_t)split * g.batch + b) * g.n + row) * g.m + col) =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                }
            }
        }
    } else {
        // bf16 results go through LDS so every global store is a full
        // 16-byte piece of a row and each 16-lane group writes a contiguous
        // 256-byte row segment.  Each wave stages its WTM x WTN block in its
        // own LDS region (rows of WTN*2 bytes, 16-byte chunk c of row r at
        // c ^ (r % CPW)), which is free of bank conflicts for both passes.
        constexpr int CPW = WTN / 8;  // 16-byte chunks per staged row
        static_assert(WTM * WTN * 2 * NW <= (int)sizeof(sA) + (int)sizeof(sB), "staging does not fit");
        static_assert((CPW & (CPW - 1)) == 0, "chunks per row must be a power of two");
        __syncthreads();  // every wave is done reading the operand tiles
        uint4 *stage = (wave * WTM * CPW < 2 * BM * 8) ? &sA[0][0] + wave * WTM * CPW
                                                      : &sB[0][0] + (wave * WTM * CPW - 2 * BM * 8);
        char *st = reinterpret_cast<char *>(stage);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = i * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c4 = j * 8 + q * 2 + (lane >> 5);  // 4-column group within the wave row
                    const uint32_t lo = pack_bf16x2(g.alpha * acc[i][j][4 * q], g.alpha * acc[i][j][4 * q + 1]);
                    const uint32_t hi = pack_bf16x2(g.alpha * acc[i][j][4 * q + 2], g.alpha * acc[i][j][4 * q + 3]);
                    const int chunk = (c4 >> 1) ^ (r & (CPW - 1));
                    *reinterpret_cast<uint2 *>(st + (r * CPW + chunk) * 16 + (c4 & 1) * 8) = make_uint2(lo, hi);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        constexpr int RPI = 64 / CPW;  // rows per pass of the wave
#pragma unroll 4
        for (int it = 0; it < WTM / RPI; ++it) {
            const int r = it * RPI + lane / CPW;
            const int c = lane % CPW;
            const uint4 v = stage[r * CPW + (c ^ (r & (CPW - 1)))];
            const int64_t row = m0 + wm * WTM + r;
            const int64_t col = n0 + wn * WTN + c * 8;
            if (row < g.n && col < g.m) *reinterpret_cast<uint4 *>(g.Y + b * g.strideY + row * g.ldy + col) = v;
        }
    }
}

// Output of a 256x256 tile computed by 4 waves of 128x128 (2x2): lane l,
// registers 4q..4q+3 of accumulator block (i, j) hold output row i*32 + l%32
// and columns j*32 + 8q + 4(l/32) + 0..3 of the wave's block.  With SPLIT the
// fp32 partials go to part[split]; otherwise the scaled bf16 results go
// through the wave's 32 KB LDS region `stage` (16-byte chunk c of row r at
// c ^ (r % 16)) so every global store is a full 16-byte piece and each
// 16-lane group writes 256 contiguous bytes of a row.  The caller has made
// sure no wave still reads operands from `stage`.
// Output of a 256x256 tile: lane l of wave (wm, wn) holds, for each
// (i, j, q), four consecutive columns n0 + 128 wn + 32 j + 8 q + 4 (l / 32)
// of row m0 + 128 wm + 32 i + l % 32.  With SPLIT the fp32 partials go to
// part[split] (alpha is applied by the reduce); otherwise the tile is
// rounded to bf16, staged in LDS and written in 16-byte row pieces.  With
// SCALED (8-bit weights) every column c is multiplied by colscale[c] too:
// the scale of the dequantized weight column, applied once to the fp32 sum.
template <bool SPLIT, bool SCALED = false>
__device__ __forceinline__ void store_tile_256(const GemmArgs &g, const f32x16_t (&acc)[4][4], uint4 *stage,
                                               int64_t m0, int64_t n0, int64_t b, int split, int wm, int wn,
                                               int lane) {
    constexpr int FM = 4, FN = 4, WTM = 128, WTN = 128;
    // factors of the four columns of (j, q): alpha (not with SPLIT) times the column scales
    auto factors = [&](int j, int q, float (&f)[4]) {
        const float a = SPLIT ? 1.f : g.alpha;
        if constexpr (SCALED) {
            const int64_t col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
            const float4 v = col < g.m ? *reinterpret_cast<const float4 *>(g.colscale + col)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
            f[0] = a * v.x;
            f[1] = a * v.y;
            f[2] = a * v.z;
            f[3] = a * v.w;
        } else {
            f[0] = f[1] = f[2] = f[3] = a;
        }
    };
    if constexpr (SPLIT) {
        (void)stage;
        if constexpr (SCALED) {
            // scale loads per (j, q), reused over the four row blocks
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
                    if (col >= g.m) continue;  // m % 8 == 0: the four columns are all in or all out
                    float f[4];
                    factors(j, q, f);
#pragma unroll
                    for (int i = 0; i < FM; ++i) {
                        const int64_t row = m0 + wm * WTM + i * 32 + (lane & 31);
                        if (row >= g.n) continue;
                        *reinterpret_cast<float4 *>(g.part + (((int64_t)split * g.batch + b) * g.n + row) * g.m + col) =
                            make_float4(f[0] * acc[i][j][4 * q], f[1] * acc[i][j][4 * q + 1],
                                        f[2] * acc[i][j][4 * q + 2], f[3] * acc[i][j][4 * q + 3]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int64_t row = m0 + wm * WTM + i * 32 + (lane & 31);
                if (row >= g.n) continue;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
                        if (col >= g.m) continue;  // m % 8 == 0: the four columns are all in or all out
                        *reinterpret_cast<float4 *>(g.part + (((int64_t)split * g.batch + b) * g.n + row) * g.m +
                                                    col) =
                            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                        acc[i][j][4 * q + 3]);
                    }
                }
            }
        }
    } else {
        constexpr int CPW = WTN / 8;
        char *st = reinterpret_cast<char *>(stage);
        auto stage_one = [&](int i, int j, int q, const float (&f)[4]) {
            const int r = i * 32 + (lane & 31);
            const int c4 = j * 8 + q * 2 + (lane >> 5);
            const uint32_t lo = pack_bf16x2(f[0] * acc[i][j][4 * q], f[1] * acc[i][j][4 * q + 1]);
            const uint32_t hi = pack_bf16x2(f[2] * acc[i][j][4 * q + 2], f[3] * acc[i][j][4 * q + 3]);
            const int chunk = (c4 >> 1) ^ (r & (CPW - 1));
            *reinterpret_cast<uint2 *>(st + (r * CPW + chunk) * 16 + (c4 & 1) * 8) = make_uint2(lo, hi);
        };
        if constexpr (SCALED) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float f[4];
                    factors(j, q, f);
#pragma unroll
                    for (int i = 0; i < FM; ++i) stage_one(i, j, q, f);
                }
        } else {
            const float f[4] = {g.alpha, g.alpha, g.alpha, g.alpha};
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) stage_one(i, j, q, f);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        constexpr int RPI = 64 / CPW;
#pragma unroll 4
        for (int it = 0; it < WTM / RPI; ++it) {
            const int r = it * RPI + lane / CPW;
            const int c = lane % CPW;
            const uint4 v = stage[r * CPW + (c ^ (r & (CPW - 1)))];
            const int64_t row = m0 + wm * WTM + r;
            const int64_t col = n0 + wn * WTN + c * 8;
            if (row < g.n && col < g.m) *reinterpret_cast<uint4 *>(g.Y + b * g.strideY + row * g.ldy + col) = v;
        }
    }
}

// SwiGLU epilogue of a 256x256 tile whose B columns interleave gate and up
// weights in 32-column blocks (launch_gated_weights): a wave's column blocks
// j = 0, 2 are gate and j = 1, 3 the matching up columns, so lane l holds
// gate and up of the same four outputs in acc[i][2jj] and acc[i][2jj + 1].
// Each wave forms h = SiLU(gate) * up, rounded to bf16, for its 128 rows x
// 64 outputs (columns 128 tn + 64 wn ..) and, through its LDS region,
//  * writes h row-major to Y when Y is given (16-byte chunk c of staged row
//    r at c ^ (r % 8); 16 stores of 8 rows x 128 bytes), and
//  * writes h^T to Yt when Yt is given (staged as 64 rows of the wave's 128
//    h rows, 136 elements apart; 16 stores of 4 rows x 256 bytes), with the
//    sums of squares of the bf16 values of each column over the wave's rows
//    below n, in row order; the wave of the lower 128 rows adds its sums to
//    those of the upper wave (through `xch`, 128 floats of LDS) and writes
//    npart[256-row chunk][column]: the column norms of h for the next
//    projection's selection, without another pass.  Every wave of the
//    workgroup must call this (it holds a workgroup barrier).
__device__ __forceinline__ float silu_f32(float z) { return z / (1.f + __expf(-z)); }

__device__ __forceinline__ void store_tile_swiglu(const GemmArgs &g, const f32x16_t (&acc)[4][4], uint4 *stage,
                                                  float *xch, int64_t m0, int64_t hcol0, int tm, int wm, int wn,
                                                  int lane) {
    constexpr int CPW = 8;  // 16-byte chunks per staged row (64 outputs)
    const int64_t mh = g.m / 2;
    uint32_t hp[4][2][4][2];  // [i][jj][q][half]: bf16 pairs of h
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[e] = silu_f32(g.alpha * acc[i][2 * jj][4 * q + e]) * (g.alpha * acc[i][2 * jj + 1][4 * q + e]);
                hp[i][jj][q][0] = pack_bf16x2(h[0], h[1]);
                hp[i][jj][q][1] = pack_bf16x2(h[2], h[3]);
            }
    char *st = reinterpret_cast<char *>(stage);
    if (g.Y) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 32 + (lane & 31);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c4 = jj * 8 + q * 2 + (lane >> 5);
                    const int chunk = (c4 >> 1) ^ (r & (CPW - 1));
                    *reinterpret_cast<uint2 *>(st + (r * CPW + chunk) * 16 + (c4 & 1) * 8) =
                        make_uint2(hp[i][jj][q][0], hp[i][jj][q][1]);
                }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int r = it * 8 + lane / CPW;
            const int c = lane % CPW;
            const uint4 v = stage[r * CPW + (c ^ (r & (CPW - 1)))];
            const int64_t row = m0 + wm * 128 + r;
            const int64_t col = hcol0 + c * 8;
            if (row < g.n && col < mh) *reinterpret_cast<uint4 *>(g.Y + row * g.ldy + col) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // the region's reads are done before it is rewritten
        __builtin_amdgcn_wave_barrier();
    }
    if (g.Yt) {
        constexpr int TS = 136;  // staged h^T row: 128 values + 8 of padding (272 bytes)
        uint16_t *t = reinterpret_cast<uint16_t *>(stage);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 32 + (lane & 31);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = jj * 32 + q * 8 + 4 * (lane >> 5);  // first of this lane's four columns
                    t[(c + 0) * TS + r] = (uint16_t)(hp[i][jj][q][0] & 0xffffu);
                    t[(c + 1) * TS + r] = (uint16_t)(hp[i][jj][q][0] >> 16);
                    t[(c + 2) * TS + r] = (uint16_t)(hp[i][jj][q][1] & 0xffffu);
                    t[(c + 3) * TS + r] = (uint16_t)(hp[i][jj][q][1] >> 16);
                }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const int64_t r0 = m0 + wm * 128;
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int c = it * 4 + lane / 16;  // staged h^T row = h column within the wave's 64
            const int ch = lane % 16;          // 16-byte chunk of the 128 rows
            const uint4 v = *reinterpret_cast<const uint4 *>(t + c * TS + ch * 8);
            const int64_t col = hcol0 + c, row = r0 + ch * 8;
            if (col < mh && row < g.n) *reinterpret_cast<uint4 *>(g.Yt + col * g.n + row) = v;  // n % 8 == 0
        }
        // column sums of squares, one column per lane, rows in order
        const int nrows = (int)max((int64_t)0, min((int64_t)128, g.n - r0));
        const uint16_t *tc = t + lane * TS;
        float sq = 0.f;
        for (int r8 = 0; r8 < nrows; r8 += 8) {  // nrows % 8 == 0
            const uint4 v = *reinterpret_cast<const uint4 *>(tc + r8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
                sq = fmaf(lo, lo, sq);
                sq = fmaf(hi, hi, sq);
            }
        }
        // the tile's 256 rows in order: rows 0..127 (wave wm = 0), then 128..255
        if (wm == 1) xch[wn * 64 + lane] = sq;
        __syncthreads();
        if (wm == 0 && hcol0 + lane < mh) g.npart[(int64_t)tm * mh + hcol0 + lane] = sq + xch[wn * 64 + lane];
    }
}

// The kept-row list of a workgroup's K range into LDS as 16-bit row numbers
// (0xffff for -1 entries and list padding, whose rows then read as zero):
// entries [0, nvalid) from src, the rest up to nlist (rounded up to a
// multiple of 4) padding.  16-byte loads of four entries, four per thread in
// flight before the first store, so the list costs one memory round trip per
// 16 NT entries instead of one per entry.  nvalid > 0; src is 16-byte aligned
// and readable up to nvalid rounded up to a multiple of 4.  Every load is
// unconditional (pieces past nvalid load piece 0 and are replaced), so the
// one wait before the stores covers all four.
template <int NT>
__device__ __forceinline__ void load_row_list(const int32_t *__restrict__ src, int nvalid, int nlist, uint16_t *dst,
                                              int tid) {
    const int nch = (nlist + 3) / 4;
    for (int base = 0; base < nch; base += 4 * NT) {
        int4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ch = base + u * NT + tid;
            q[u] = *reinterpret_cast<const int4 *>(src + (ch * 4 < nvalid ? ch * 4 : 0));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ch = base + u * NT + tid;
            const int t = ch * 4;
            const uint32_t e0 = (t >= nvalid || q[u].x < 0) ? 0xffffu : (uint32_t)q[u].x;
            const uint32_t e1 = (t + 1 >= nvalid || q[u].y < 0) ? 0xffffu : (uint32_t)q[u].y;
            const uint32_t e2 = (t + 2 >= nvalid || q[u].z < 0) ? 0xffffu : (uint32_t)q[u].z;
            const uint32_t e3 = (t + 3 >= nvalid || q[u].w < 0) ? 0xffffu : (uint32_t)q[u].w;
            if (ch < nch) *reinterpret_cast<uint2 *>(dst + t) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
        }
    }
}

// Reduced product with A fragments loaded straight from HBM into registers
// (256x256 output tile, 4 waves in a 2x2 grid, each wave 128x128).
//
// A[:, I] arrives packed in MFMA operand order (pack_kernel, layout 1): the
// operand of one 32x32x16 step for 32 rows and 16 kept indices is a 1 KB
// block in which lane l's 16 bytes hold row l % 32, entries 8 (l / 32) ..
// +7.  Block (row block R, 16-entry group G) sits at (R * kpad/16 + G) KB.
// Every A fragment is therefore one coalesced 16-byte-per-lane load, issued
// two K steps before its MFMAs into the register slot its previous contents
// just left; A never passes through LDS.
//
// Only the gathered rows of B go through LDS: per K step, each thread loads
// eight 16-byte pieces (eight kept rows x 8 columns) through the index list
// two steps ahead, stores the previous step's pieces into the free LDS
// buffer over sub-steps 0-2 and the waves read their MFMA operands with
// ds_read_b64_tr_b16 (row-major B tile: chunk c of row k at c ^ 2(k & 3)).
// The kept row numbers of the workgroup's K range are copied once into LDS
// as 16-bit values (0xffff marks padding: such rows read as zero), so the
// gather never waits on a global index load.
template <bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_adirect_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, NT = 256, WTM = 128, WTN = 128;
    constexpr int FM = 4, FN = 4;
    constexpr int CPR = BN / 8;        // 16-byte chunks per B row
    constexpr int BUF = BK * CPR;      // uint4 per B buffer (32 KB)
    __shared__ uint4 sL[4 * BUF];      // B buffers 0/1 | kept row numbers (u16, 64 KB) ; epilogue staging
    uint16_t *sIdx = reinterpret_cast<uint16_t *>(sL + 2 * BUF);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
    const int tiles_m = (int)((g.n + BM - 1) / BM), tiles_n = (int)((g.m + BN - 1) / BN);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t b = blockIdx.z;
    const int split = blockIdx.y;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + b * g.strideA, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (b / g.group) * g.strideB, g.b_bytes);
    const int32_t *idx = g.idx + b * g.ld_idx;

    const int KT = (int)(g.kpad / BK);
    const int per = ((KT + g.splits - 1) / g.splits + 1) & ~1;
    const int kt0 = split * per;
    const int kt1 = min(KT, kt0 + per);
    const int KG = (int)(g.kpad / 16);

    // this wave's A row blocks; blocks past n read as zero
    uint32_t aoff[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t rb = (m0 + wm * WTM) / 32 + i;
        aoff[i] = rb * 32 < g.n ? (uint32_t)(rb * KG * 1024 + lane * 16) : kOob;
    }
    // B: thread owns kept rows kq*8 .. kq*8+7 of a step, 16-byte column chunk nc
    const int kq = tid / CPR, nc = tid % CPR;
    const uint32_t ldb2 = (uint32_t)(g.ldb * 2), bcol2 = (uint32_t)((n0 + nc * 8) * 2);

    auto load_rows = [&](int kt, uint32_t (&o)[4]) {  // eight u16 row numbers, one LDS read
        const int t0 = (min(kt, kt1 - 1) - kt0) * BK + kq * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(sIdx + t0);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    };
    auto load_b = [&](int r0, int r1, uint4 (&rb)[8], const uint32_t (&ix)[4]) {
#pragma unroll
        for (int r = r0; r < r1; ++r) {
            const uint32_t row = (r & 1) ? (ix[r >> 1] >> 16) : (ix[r >> 1] & 0xffffu);
            rb[r] = buf_load16(rB, row == 0xffffu ? kOob : row * ldb2 + bcol2);
        }
    };
    auto load_a = [&](int kt, int ks, bf16x8_t (&fa)[FM]) {
        const uint32_t ko = (uint32_t)(min(kt, kt1 - 1) * 4 + ks) * 1024u;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = as_bf16x8(buf_load16(rA, aoff[i] + ko));
    };
    auto store_b = [&](int buf, const uint4 (&rb)[8], int r0, int r1) {
#pragma unroll
        for (int r = r0; r < r1; ++r) {
            const int k = kq * 8 + r;
            sL[buf * BUF + k * CPR + (nc ^ ((k & 3) << 1))] = rb[r];
        }
    };
    auto read_b = [&](int buf, int ks, bf16x8_t (&fb)[FN]) {
        const int gq = lane >> 4, li = lane & 15;
        const int kbase = ks * 16 + 8 * (gq >> 1) + (li >> 2);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int nn = wn * WTN + j * 32 + 16 * (gq & 1) + 4 * (li & 3);
            union {
                v4i16_t h[2];
                bf16x8_t v;
            } u;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int k = kbase + 4 * hh;
                const char *p = reinterpret_cast<const char *>(&sL[buf * BUF + k * CPR + ((nn >> 3) ^ ((k & 3) << 1))]) +
                                ((nn >> 2) & 1) * 8;
                u.h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)p);
            }
            fb[j] = u.v;
        }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    bf16x8_t fa[2][4][FM];  // [step parity][sub-step][row block]
    bf16x8_t fb[2][FN];
    uint4 rb0[8], rb1[8];
    uint32_t ix0[4], ix1[4];

    // one K step on LDS buffer `buf` and A slot set `p`: B rows of step kt+2
    // are loaded into lb while those of step kt+1 (sb) are stored
    auto step = [&](int kt, int p, int buf, uint4 (&lb)[8], uint32_t (&lix)[4], const uint4 (&sb)[8]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) read_b(buf, ks + 1, fb[(ks + 1) & 1]);
            else read_b(buf ^ 1, 0, fb[0]);
            if (ks < 3) {
                load_b(ks * 3, min(8, ks * 3 + 3), lb, lix);
                store_b(buf ^ 1, sb, ks * 3, min(8, ks * 3 + 3));
            }
            // operands swapped: each lane ends up holding four consecutive
            // output columns of one output row
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[p][ks][i], acc[i][j], 0, 0, 0);
            load_a(kt + 2, ks, fa[p][ks]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 2) __syncthreads();
        }
        load_rows(kt + 4, lix);
    };

    if (kt0 < kt1) {
        load_row_list<NT>(idx + kt0 * BK, (kt1 - kt0) * BK, (kt1 - kt0) * BK, sIdx, tid);
        __syncthreads();
        load_rows(kt0, ix0);
        load_rows(kt0 + 1, ix1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) load_a(kt0, ks, fa[0][ks]);
        load_b(0, 8, rb0, ix0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) load_a(kt0 + 1, ks, fa[1][ks]);
        load_b(0, 8, rb1, ix1);
        load_rows(kt0 + 2, ix0);
        load_rows(kt0 + 3, ix1);
        store_b(0, rb0, 0, 8);
        __syncthreads();
        read_b(0, 0, fb[0]);
        for (int kt = kt0; kt < kt1; kt += 2) {
            step(kt, 0, 0, rb0, ix0, rb1);      // step kt on buffer 0; step kt+1's rows -> buffer 1
            step(kt + 1, 1, 1, rb1, ix1, rb0);  // step kt+1 on buffer 1; step kt+2's rows -> buffer 0
        }
    }

    __syncthreads();  // every wave is done with the operand buffers
    store_tile_256<SPLIT>(g, acc, sL + w * WTM * (WTN / 8), m0, n0, b, split, wm, wn, lane);
}

// Reduced product with A fragments loaded straight into registers and the
// gathered B rows copied into LDS by the load unit itself (buffer loads with
// the LDS-destination bit: no registers, no LDS store instructions).
//
// Tile, waves, A handling and the u16 kept-row list are those of
// gemm_adirect_kernel; what changes is the path of B.  Each K step's 64 x 256
// B tile sits in one of three LDS stages.  During sub-steps 0-1 of step kt
// every wave issues eight 1 KB LDS-DMA loads for step kt+2 (its 16 tile rows:
// lanes 0-31 fetch one kept row's 512 bytes, lanes 32-63 the next, each lane
// the 16-byte chunk that belongs at its position under the chunk ^ 2(k & 3)
// swizzle that ds_read_b64_tr_b16 reads conflict-free).  After sub-step 2
// each wave waits until its own loads of step kt+1 have landed and the
// workgroup barrier publishes that stage; sub-step 3 then already reads the
// first operands of step kt+1.  A fragments of step kt+1 are loaded into each
// sub-step's registers as its MFMAs release them (one step ahead).
//
// The three stages are separate LDS arrays addressed at compile time (the
// loop is unrolled by three), so the compiler can tell the stage being
// filled from the stages being read and only waits where the data is needed.
// Vector-memory loads complete in issue order: when a wave waits after
// sub-step 2 of step kt, at least 28 loads were issued after its last DMA
// load of step kt+1 (the A loads of sub-steps 2-3 of step kt-1, then 8 DMA
// and 12 A loads of step kt, each group fenced by a scheduling barrier), so
// vmcnt(28) covers it.  The K range of a workgroup is rounded up to whole
// groups of three steps; the added steps read the padding entry (0xffff) for
// every B row and out-of-range offsets for A, so they add exact zeros.
template <bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_bdma_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, WTM = 128, WTN = 128;
    constexpr int FM = 4, FN = 4;
    constexpr int CPR = BN / 8;    // 16-byte chunks per B row
    constexpr int BUF = BK * CPR;  // uint4 per B stage (32 KB)
    __shared__ uint4 sB0[BUF];
    __shared__ uint4 sB1[BUF];
    __shared__ uint4 sB2[BUF];
    __shared__ uint4 sX[BUF];  // kept row numbers (u16, kBdmaListRows); wave 3's epilogue staging
    uint16_t *sIdx = reinterpret_cast<uint16_t *>(sX);
    typedef __attribute__((address_space(3))) void lds_t;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
    const int tiles_m = (int)((g.n + BM - 1) / BM), tiles_n = (int)((g.m + BN - 1) / BN);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t b = blockIdx.z;
    const int split = blockIdx.y;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + b * g.strideA, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (b / g.group) * g.strideB, g.b_bytes);
    const int32_t *idx = g.idx + b * g.ld_idx;

    // the split boundaries are those of gemm_adirect_kernel
    const int KT = (int)(g.kpad / BK);
    const int per = ((KT + g.splits - 1) / g.splits + 1) & ~1;
    const int kt0 = split * per;
    const int kt1 = min(KT, kt0 + per);
    const int kte = kt0 + (max(kt1 - kt0, 0) + 2) / 3 * 3;  // end of the padded range
    const int KG = (int)(g.kpad / 16);

    uint32_t aoff[FM];  // this wave's A row blocks; blocks past n read as zero
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t rb = (m0 + wm * WTM) / 32 + i;
        aoff[i] = rb * 32 < g.n ? (uint32_t)(rb * KG * 1024 + lane * 16) : kOob;
    }
    const uint32_t ldb2 = (uint32_t)(g.ldb * 2), nb2 = (uint32_t)(n0 * 2);
    const int hsel = lane >> 5, pos = lane & 31;

    // row numbers of this wave's tile rows 16w .. 16w+15 of step kt (two
    // broadcast 16-byte LDS reads); lane keeps rows 16w + 2i + hsel
    auto load_rows = [&](int kt, uint32_t (&o)[8]) {
        const int t0 = (kt - kt0) * BK + 16 * w;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(sIdx + t0);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(sIdx + t0 + 8);
        const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = hsel ? (wd[i] >> 16) : (wd[i] & 0xffffu);
    };
    // LDS-DMA loads i0..i1-1 into stage dst: load i fills tile rows 16w + 2i
    // (lanes 0-31) and 16w + 2i + 1 (lanes 32-63); lane position p of row kr
    // holds logical chunk p ^ 2(kr & 3)
    auto dma_b = [&](uint4 *dst, int i0, int i1, const uint32_t (&rows)[8]) {
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            const int kr = 16 * w + 2 * i + hsel;
            const uint32_t c = (uint32_t)(pos ^ ((kr & 3) << 1));
            const uint32_t row = rows[i];
            // padding rows (0xffff) get the out-of-range bit (a select, not a branch)
            const uint32_t off = (row * ldb2 + nb2 + c * 16u) | (row == 0xffffu ? kOob : 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_t *)&dst[(16 * w + 2 * i) * CPR], 16, off, 0, 0, 0);
        }
    };
    auto load_a = [&](int kt, int ks, bf16x8_t (&fa)[FM]) {
        const bool live = kt < kt1;  // steps of the padded range read zeros
        const uint32_t ko = (uint32_t)(kt * 4 + ks) * 1024u;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = as_bf16x8(buf_load16(rA, live ? aoff[i] + ko : kOob));
    };
    auto read_b = [&](const uint4 *stg, int ks, bf16x8_t (&fb)[FN]) {
        const int gq = lane >> 4, li = lane & 15;
        const int kbase = ks * 16 + 8 * (gq >> 1) + (li >> 2);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int nn = wn * WTN + j * 32 + 16 * (gq & 1) + 4 * (li & 3);
            union {
                v4i16_t h[2];
                bf16x8_t v;
            } u;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int k = kbase + 4 * hh;
                const char *p = reinterpret_cast<const char *>(&stg[k * CPR + ((nn >> 3) ^ ((k & 3) << 1))]) +
                                ((nn >> 2) & 1) * 8;
                u.h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)p);
            }
            fb[j] = u.v;
        }
    };
    auto stage_of = [&](auto Sc) -> uint4 * {
        constexpr int S = decltype(Sc)::value % 3;
        if constexpr (S == 0) return sB0;
        else if constexpr (S == 1) return sB1;
        else return sB2;
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    bf16x8_t fa[4][FM];  // [sub-step][row block]
    bf16x8_t fb[2][FN];
    uint32_t rows[8];

    // one K step on stage S (S + 1 holds step kt+1, S + 2 receives kt+2)
    auto step = [&](int kt, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const uint4 *cur = stage_of(std::integral_constant<int, S>{});
        const uint4 *nxt1 = stage_of(std::integral_constant<int, S + 1>{});
        uint4 *nxt2 = stage_of(std::integral_constant<int, S + 2>{});
        load_rows(kt + 2, rows);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) read_b(cur, ks + 1, fb[(ks + 1) & 1]);
            else read_b(nxt1, 0, fb[0]);
            if (ks < 2) dma_b(nxt2, 4 * ks, 4 * ks + 4, rows);
            // operands swapped: each lane ends up holding four consecutive
            // output columns of one output row
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks][i], acc[i][j], 0, 0, 0);
            load_a(kt + 1, ks, fa[ks]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 2) {
                __builtin_amdgcn_s_waitcnt(0x407c);  // vmcnt(28) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (kt0 < kt1) {
        // list entries for the padded range plus the two steps loaded past it
        const int nlist = (kte - kt0 + 2) * BK;  // <= kBdmaListRows (checked by the host)
        load_row_list<256>(idx + kt0 * BK, (kt1 - kt0) * BK, nlist, sIdx, tid);
        __syncthreads();
        load_rows(kt0, rows);
        dma_b(sB0, 0, 8, rows);
        load_rows(kt0 + 1, rows);
        dma_b(sB1, 0, 8, rows);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) load_a(kt0, ks, fa[ks]);
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): stages 0 and 1 are complete
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_b(sB0, 0, fb[0]);
        for (int kt = kt0; kt < kte; kt += 3) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
            step(kt + 2, std::integral_constant<int, 2>{});
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS-DMA load still writing when the stages are reused
    __syncthreads();
    uint4 *stage = w == 0 ? sB0 : w == 1 ? sB1 : w == 2 ? sB2 : sX;
    store_tile_256<SPLIT>(g, acc, stage, m0, n0, b, split, wm, wn, lane);
}

// Eight 8-bit weight codes (k-consecutive, as ds_read_b64_tr_b8 delivers
// them for one column) widened to the bf16 MFMA operand.  Both formats are
// exact in bf16: an E4M3 value has at most 4 significant bits and an
// exponent in [-9, 8]; an int8 value at most 8 significant bits.  FP8 uses
// gfx950's packed conversion (scale 1); int8 converts each sign-extended
// byte to fp32 and packs pairs (round-to-nearest-even, exact here).
template <int BQ>
__device__ __forceinline__ bf16x8_t codes_to_bf16x8(uint32_t lo, uint32_t hi) {
    if constexpr (BQ == 1) {
        const rmm_bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
        const rmm_bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
        const rmm_bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
        const rmm_bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
        return as_bf16x8(make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)));
    } else {
        const int32_t x = (int32_t)lo, y = (int32_t)hi;
        return as_bf16x8(make_uint4(
            pack_bf16x2((float)(int8_t)x, (float)(int8_t)(x >> 8)), pack_bf16x2((float)(int8_t)(x >> 16), (float)(x >> 24)),
            pack_bf16x2((float)(int8_t)y, (float)(int8_t)(y >> 8)), pack_bf16x2((float)(int8_t)(y >> 16), (float)(y >> 24))));
    }
}

// Reduced product with both operands gathered by rows through LDS: A^T
// (the activation block transposed, d x n, written by the column-norm pass)
// supplies rows A^T[I_t, :] exactly as B supplies rows B[I_t, :], so neither
// operand needs a separate pack pass.
//
// Tile and waves are those of gemm_bdma_kernel (256x256, four waves of
// 128x128).  Each K step's 64 x 256 tiles of both operands sit in one of two
// LDS stages per operand (4 x 32 KB), filled by LDS-DMA buffer loads in the
// layout ds_read_b64_tr_b16 reads conflict-free (chunk c of row k at
// c ^ 2(k & 3)); the transposed reads give the A fragments the same
// per-lane layout as the B fragments (eight consecutive k of one row), the
// layout the operand blocks of gemm_adirect_kernel hold.  One barrier per
// step, after sub-step 2: every wave waits for its own loads of step kt+1
// (vmcnt(0): the LDS-DMA loads are its only vector-memory loads), and the
// barrier both publishes stage kt+1 and certifies that every wave has read
// its last operands of stage kt (sub-step 3's fragments were read during
// sub-step 2).  The loads are spread over two sub-steps, eight per wave in
// each, interleaved with the MFMAs: sub-step 3 of step kt refills the A
// stage of step kt with step kt+2 (a step and a quarter to land) and
// sub-step 0 of step kt fills the B stage of step kt+1, free since the
// barrier of step kt-1 (three quarters of a step).  Issuing all sixteen in
// sub-step 3 measured 4-5% slower on MI355X.  The kept row list lives in LDS
// as 16-bit numbers (kTdmaListRows entries per split, 0xffff for padding:
// such rows read as zero).  Per K step it is as fast as the A-direct kernel
// on a 4096 x 4096 x 4096 projection and 2-4% faster than gemm_bdma_kernel
// on a 2048 x 14336 x 4096 one, without the pack pass either needs.
template <bool SPLIT, int EPI, int BQ = 0>
__global__ __launch_bounds__(256, 1) void gemm_tdma_kernel(GemmArgs g) {
    static_assert(BQ == 0 || EPI == 0, "8-bit weights with the plain epilogue only");
    constexpr int BM = 256, BN = 256, WTM = 128, WTN = 128;
    constexpr int FM = 4, FN = 4;
    constexpr int CPR = 32;
    constexpr int BUF = BK * CPR;  // uint4 per stage (32 KB)
    // 8-bit B: 64 rows x 256 codes per stage (16 KB); the list then takes the
    // LDS left (64 KB), which also stages waves 2 and 3 in the epilogue.
    // Separate arrays, so the compiler can tell the LDS-DMA writes of one
    // stage from the reads of another and need not wait between them.
    constexpr int BUFB = BQ ? BUF / 2 : BUF;
    __shared__ uint4 sA0[BUF];
    __shared__ uint4 sA1[BUF];
    __shared__ uint4 sB0[BUFB];
    __shared__ uint4 sB1[BUFB];
    __shared__ __align__(16) uint16_t sIdx[BQ ? kTdmaListRowsQ : kTdmaListRows];
    typedef __attribute__((address_space(3))) void lds_t;

    // the wave index is uniform: from an SGPR, LDS-DMA destinations (M0) are scalar arithmetic
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 1,
              wn = w & 1;
    const int tiles_m = (int)((g.n + BM - 1) / BM), tiles_n = (int)((g.m + BN - 1) / BN);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t b = blockIdx.z;
    const int split = blockIdx.y;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + b * g.strideA, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (b / g.group) * g.strideB, g.b_bytes);
    const int32_t *idx = g.idx + b * g.ld_idx;

    const int KT = (int)(g.kpad / BK);
    const int per = ((KT + g.splits - 1) / g.splits + 1) & ~1;
    const int kt0 = split * per;
    const int kt1 = min(KT, kt0 + per);
    const int kte = kt0 + (max(kt1 - kt0, 0) + 1) / 2 * 2;
    const uint32_t lda2 = (uint32_t)(g.lda * 2), ma2 = (uint32_t)(m0 * 2);
    constexpr uint32_t BE = BQ ? 1u : 2u;  // bytes per B element
    const uint32_t ldb2 = (uint32_t)(g.ldb * BE), nb2 = (uint32_t)(n0 * BE);
    const int hsel = lane >> 5, pos = lane & 31;

    auto load_rows = [&](int kt, uint32_t (&o)[8]) {
        const int t0 = (kt - kt0) * BK + 16 * w;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(sIdx + t0);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(sIdx + t0 + 8);
        const uint32_t wd[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = hsel ? (wd[i] >> 16) : (wd[i] & 0xffffu);
    };
    auto dma = [&](__amdgpu_buffer_rsrc_t rs, uint32_t ld2, uint32_t c2, uint4 *dst, int i0, int i1,
                   const uint32_t (&rows)[8]) {
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            const int kr = 16 * w + 2 * i + hsel;
            const uint32_t c = (uint32_t)(pos ^ ((kr & 3) << 1));
            const uint32_t row = rows[i];
            const uint32_t off = (row * ld2 + c2 + c * 16u) | (row == 0xffffu ? kOob : 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t *)&dst[(16 * w + 2 * i) * CPR], 16, off, 0, 0, 0);
        }
    };
    auto read_tr = [&](const uint4 *stg, int ks, int base, bf16x8_t (&f)[4]) {
        const int gq = lane >> 4, li = lane & 15;
        const int kbase = ks * 16 + 8 * (gq >> 1) + (li >> 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nn = base + j * 32 + 16 * (gq & 1) + 4 * (li & 3);
            union {
                v4i16_t h[2];
                bf16x8_t v;
            } u;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int k = kbase + 4 * hh;
                const char *p = reinterpret_cast<const char *>(&stg[k * CPR + ((nn >> 3) ^ ((k & 3) << 1))]) +
                                ((nn >> 2) & 1) * 8;
                u.h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)p);
            }
            f[j] = u.v;
        }
    };
    // 8-bit B: a stage holds the step's 64 kept rows x 256 codes (16 KB), the
    // 16-byte chunk c of row k at c ^ (k & 7).  A wave fills 16 rows with four
    // LDS-DMA loads of 1 KB (four rows each: lane l fetches chunk
    // (l & 15) ^ (k & 7) of row 4i + l / 16 of its 16).
    auto load_rows_q = [&](int kt, uint32_t (&o)[4]) {
        const int t0 = (kt - kt0) * BK + 16 * w;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(sIdx + t0);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(sIdx + t0 + 8);
        const int gg = lane >> 4;  // entry 4i + gg of the wave's 16
        const uint32_t sh = (gg & 1) ? 16u : 0u;
        o[0] = ((gg >> 1) ? v0.y : v0.x) >> sh & 0xffffu;
        o[1] = ((gg >> 1) ? v0.w : v0.z) >> sh & 0xffffu;
        o[2] = ((gg >> 1) ? v1.y : v1.x) >> sh & 0xffffu;
        o[3] = ((gg >> 1) ? v1.w : v1.z) >> sh & 0xffffu;
    };
    auto dma_q = [&](uint4 *dst, const uint32_t (&r4)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = 16 * w + 4 * i + (lane >> 4);
            const uint32_t c = (uint32_t)((lane & 15) ^ (kr & 7));
            const uint32_t row = r4[i];
            const uint32_t off = (row * ldb2 + nb2 + c * 16u) | (row == 0xffffu ? kOob : 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_t *)&dst[(16 * w + 4 * i) * 16], 16, off, 0, 0, 0);
        }
    };
    // B fragments of sub-step ks from an 8-bit stage: one transposed 8-byte
    // read per fragment (lane i of a 16-lane group addresses row i / 2, eight
    // columns 8 (i & 1) of the group's 16; lane j then holds column j's eight
    // codes), the raw codes kept for codes_to_bf16x8
    auto read_q = [&](const uint4 *stg, int ks, int base, uint2 (&f)[4]) {
        const int gq = lane >> 4, li = lane & 15;
        const int k = ks * 16 + 8 * (gq >> 1) + (li >> 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = base + j * 32 + 16 * (gq & 1) + 8 * (li & 1);
            const char *p = reinterpret_cast<const char *>(stg) + k * 256 + (((col >> 4) ^ (k & 7)) << 4) + (col & 15);
            typedef int v2i_t __attribute__((ext_vector_type(2)));
            const v2i_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_t *)p);
            f[j] = make_uint2((uint32_t)v.x, (uint32_t)v.y);
        }
    };
    auto stA = [&](auto Sc) -> uint4 * {
        if constexpr (decltype(Sc)::value % 2 == 0) return sA0; else return sA1;
    };
    auto stB = [&](auto Sc) -> uint4 * {
        if constexpr (decltype(Sc)::value % 2 == 0) return sB0; else return sB1;
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    bf16x8_t fa[2][FM], fb[2][FN];
    uint2 fq[2][FN];  // 8-bit B: raw codes of the fragments
    uint32_t rows[8];

    auto step = [&](int kt, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const uint4 *cA = stA(std::integral_constant<int, S>{});
        const uint4 *cB = stB(std::integral_constant<int, S>{});
        const uint4 *oA = stA(std::integral_constant<int, S + 1>{});
        const uint4 *oB = stB(std::integral_constant<int, S + 1>{});
        uint4 *dA = stA(std::integral_constant<int, S>{});        // receives A of step kt+2
        uint4 *dB = stB(std::integral_constant<int, S + 1>{});    // receives B of step kt+1
        uint32_t next[8];  // rows of step kt+1
#pragma unroll
        for (int i = 0; i < 8; ++i) next[i] = rows[i];
        load_rows(kt + 2, rows);
        uint32_t nextq[4];  // 8-bit B: rows of step kt+1 in the layout of dma_q
        if constexpr (BQ != 0) load_rows_q(kt + 1, nextq);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) {
                if constexpr (BQ != 0)
                    read_q(cB, ks + 1, wn * WTN, fq[(ks + 1) & 1]);
                else
                    read_tr(cB, ks + 1, wn * WTN, fb[(ks + 1) & 1]);
                read_tr(cA, ks + 1, wm * WTM, fa[(ks + 1) & 1]);
            } else {
                if constexpr (BQ != 0)
                    read_q(oB, 0, wn * WTN, fq[0]);
                else
                    read_tr(oB, 0, wn * WTN, fb[0]);
                read_tr(oA, 0, wm * WTM, fa[0]);
            }
            if (ks == 0) {
                if constexpr (BQ != 0)
                    dma_q(dB, nextq);
                else
                    dma(rB, ldb2, nb2, dB, 0, 8, next);
            }
            if (ks == 3) dma(rA, lda2, ma2, dA, 0, 8, rows);
            if constexpr (BQ != 0) {
                // fragment j widened just before its four MFMAs
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const bf16x8_t bj = codes_to_bf16x8<BQ>(fq[ks & 1][j].x, fq[ks & 1][j].y);
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bj, fa[ks & 1][i], acc[i][j], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
            }
            if constexpr (BQ != 0) {
                // per MFMA: the conversions of the next fragment, an LDS read, and in
                // sub-steps 0 and 3 an LDS-DMA load (four of B in 0, eight of A in 3)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, BQ == 1 ? 1 : 3, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // LDS read
                    if (ks == 3 && q < 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    if (ks == 0 && q < 4) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            } else if (ks == 0 || ks == 3) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // LDS-DMA load
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 2) {
                __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (kt0 < kt1) {
        const int nlist = (kte - kt0 + 2) * BK;
        load_row_list<256>(idx + kt0 * BK, (kt1 - kt0) * BK, nlist, sIdx, tid);
        __syncthreads();
        // steps kt0 (both operands) and kt0+1 (A; its B is loaded in step kt0's sub-step 0)
        load_rows(kt0, rows);
        dma(rA, lda2, ma2, sA0, 0, 8, rows);
        if constexpr (BQ != 0) {
            uint32_t r4[4];
            load_rows_q(kt0, r4);
            dma_q(sB0, r4);
        } else {
            dma(rB, ldb2, nb2, sB0, 0, 8, rows);
        }
        load_rows(kt0 + 1, rows);
        dma(rA, lda2, ma2, sA1, 0, 8, rows);
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BQ != 0)
            read_q(sB0, 0, wn * WTN, fq[0]);
        else
            read_tr(sB0, 0, wn * WTN, fb[0]);
        read_tr(sA0, 0, wm * WTM, fa[0]);
        for (int kt = kt0; kt < kte; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    static_assert(BQ == 0 || kTdmaListRowsQ * 2 >= 2 * BUF * 16, "the list region stages two 32 KB tiles");
    uint4 *stage = w == 0 ? sA0 : w == 1 ? sA1 : BQ ? reinterpret_cast<uint4 *>(sIdx) + (w - 2) * BUF
                                                    : w == 2 ? sB0 : sB1;
    if constexpr (EPI == 1)  // the row list is no longer read: its LDS takes the exchange of column sums
        store_tile_swiglu(g, acc, stage, reinterpret_cast<float *>(sIdx), m0, n0 / 2 + wn * 64, tm, wm, wn, lane);
    else
        store_tile_256<SPLIT, BQ != 0>(g, acc, stage, m0, n0, b, split, wm, wn, lane);
}

// Epilogue of one wave's 128 x 64 part of a 256 x 256 tile (four 32-row by
// two 32-column MFMA blocks), as store_tile_256 for the 128 x 128 parts:
// fp32 partials of Y straight to g.part under split K, else alpha times the
// sums rounded to bf16, staged in the wave's 16 KB LDS region (16-byte chunk
// c of row r at c ^ (r % 8)) and written as 128-byte row pieces.
template <bool SPLIT>
__device__ __forceinline__ void store_tile_w8(const GemmArgs &g, const f32x16_t (&acc)[4][2], uint4 *stage,
                                              int64_t m0, int64_t n0, int64_t b, int split, int wm, int wn, int lane) {
    constexpr int FM = 4, FN = 2, WTM = 128, WTN = 64, CPW = WTN / 8;
    if constexpr (SPLIT) {
        (void)stage;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t row = m0 + wm * WTM + i * 32 + (lane & 31);
            if (row >= g.n) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t col = n0 + wn * WTN + j * 32 + q * 8 + (lane >> 5) * 4;
                    if (col >= g.m) continue;  // m % 8 == 0: the four columns are all in or all out
                    *reinterpret_cast<float4 *>(g.part + (((int64_t)split * g.batch + b) * g.n + row) * g.m + col) =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                }
        }
    } else {
        char *st = reinterpret_cast<char *>(stage);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = i * 32 + (lane & 31);
                    const int c4 = j * 8 + q * 2 + (lane >> 5);
                    const uint32_t lo = pack_bf16x2(g.alpha * acc[i][j][4 * q], g.alpha * acc[i][j][4 * q + 1]);
                    const uint32_t hi = pack_bf16x2(g.alpha * acc[i][j][4 * q + 2], g.alpha * acc[i][j][4 * q + 3]);
                    const int chunk = (c4 >> 1) ^ (r & (CPW - 1));
                    *reinterpret_cast<uint2 *>(st + (r * CPW + chunk) * 16 + (c4 & 1) * 8) = make_uint2(lo, hi);
                }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        constexpr int RPI = 64 / CPW;
#pragma unroll 4
        for (int it = 0; it < WTM / RPI; ++it) {
            const int r = it * RPI + lane / CPW;
            const int c = lane % CPW;
            const uint4 v = stage[r * CPW + (c ^ (r & (CPW - 1)))];
            const int64_t row = m0 + wm * WTM + r;
            const int64_t col = n0 + wn * WTN + c * 8;
            if (row < g.n && col < g.m) *reinterpret_cast<uint4 *>(g.Y + b * g.strideY + row * g.ldy + col) = v;
        }
    }
}

// Two-operand reduced product with eight waves, the kernel for bf16 B with
// the plain or split-K epilogue (gemm_tdma_kernel's 256 x 256 tile, LDS
// stages, copy schedule and barrier protocol; gemm_tdma_kernel itself runs
// the SwiGLU epilogue and 8-bit B).  Four waves of 128 x 128 keep one wave
// per SIMD: while it waits on its fragment reads, the copies or the step
// barrier, its SIMD's matrix core idles.  Here each SIMD holds two waves of
// 128 x 64 (128 accumulator registers each), so one can issue MFMAs while
// the other waits; measured on MI355X 0.5-2.5% faster on the 70B up
// projection and a 4096^3 projection, within 1% on the split-K down
// projection, and per-wave cycle counters put 22% of each wave's loop in the
// step barrier (waves of the one workgroup arriving at different times).  Per 16-deep sub-step a wave reads four A and two B fragments (12
// transposed reads) for eight MFMAs, 1.5 reads per MFMA against 1.0 with
// 128 x 128 waves.  Wave w: rows 128 (w / 4), columns 64 (w % 4) of the
// tile; it copies rows 8w .. 8w + 7 of each K step's 64 kept rows of both
// operands (four LDS-DMA loads of two rows each per operand).
template <bool SPLIT>
__global__ __launch_bounds__(512, 1) void gemm_tdma8_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, WTM = 128, WTN = 64;
    constexpr int FM = 4, FN = 2;
    constexpr int CPR = 32;
    constexpr int BUF = BK * CPR;  // uint4 per stage (32 KB)
    __shared__ uint4 sA0[BUF];
    __shared__ uint4 sA1[BUF];
    __shared__ uint4 sB0[BUF];
    __shared__ uint4 sB1[BUF];
    __shared__ __align__(16) uint16_t sIdx[kTdmaListRows];
    typedef __attribute__((address_space(3))) void lds_t;

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w >> 2,
              wn = w & 3;
    const int tiles_m = (int)((g.n + BM - 1) / BM), tiles_n = (int)((g.m + BN - 1) / BN);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t b = blockIdx.z;
    const int split = blockIdx.y;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + b * g.strideA, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (b / g.group) * g.strideB, g.b_bytes);
    const int32_t *idx = g.idx + b * g.ld_idx;

    const int KT = (int)(g.kpad / BK);
    const int per = ((KT + g.splits - 1) / g.splits + 1) & ~1;
    const int kt0 = split * per;
    const int kt1 = min(KT, kt0 + per);
    const int kte = kt0 + (max(kt1 - kt0, 0) + 1) / 2 * 2;
    const uint32_t lda2 = (uint32_t)(g.lda * 2), ma2 = (uint32_t)(m0 * 2);
    const uint32_t ldb2 = (uint32_t)(g.ldb * 2), nb2 = (uint32_t)(n0 * 2);
    const int hsel = lane >> 5, pos = lane & 31;

    auto load_rows = [&](int kt, uint32_t (&o)[4]) {
        const int t0 = (kt - kt0) * BK + 8 * w;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(sIdx + t0);
        const uint32_t wd[4] = {v0.x, v0.y, v0.z, v0.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = hsel ? (wd[i] >> 16) : (wd[i] & 0xffffu);
    };
    auto dma = [&](__amdgpu_buffer_rsrc_t rs, uint32_t ld2, uint32_t c2, uint4 *dst, const uint32_t (&rows)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kr = 8 * w + 2 * i + hsel;
            const uint32_t c = (uint32_t)(pos ^ ((kr & 3) << 1));
            const uint32_t row = rows[i];
            const uint32_t off = (row * ld2 + c2 + c * 16u) | (row == 0xffffu ? kOob : 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t *)&dst[(8 * w + 2 * i) * CPR], 16, off, 0, 0, 0);
        }
    };
    auto read_tr = [&](const uint4 *stg, int ks, int base, bf16x8_t *f, auto NFc) {
        constexpr int NF = decltype(NFc)::value;
        const int gq = lane >> 4, li = lane & 15;
        const int kbase = ks * 16 + 8 * (gq >> 1) + (li >> 2);
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int nn = base + j * 32 + 16 * (gq & 1) + 4 * (li & 3);
            union {
                v4i16_t h[2];
                bf16x8_t v;
            } u;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int k = kbase + 4 * hh;
                const char *p = reinterpret_cast<const char *>(&stg[k * CPR + ((nn >> 3) ^ ((k & 3) << 1))]) +
                                ((nn >> 2) & 1) * 8;
                u.h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)p);
            }
            f[j] = u.v;
        }
    };
    auto stA = [&](auto Sc) -> uint4 * {
        if constexpr (decltype(Sc)::value % 2 == 0) return sA0; else return sA1;
    };
    auto stB = [&](auto Sc) -> uint4 * {
        if constexpr (decltype(Sc)::value % 2 == 0) return sB0; else return sB1;
    };
    using FMc = std::integral_constant<int, FM>;
    using FNc = std::integral_constant<int, FN>;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    bf16x8_t fa[2][FM], fb[2][FN];
    uint32_t rows[4];

    auto step = [&](int kt, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const uint4 *cA = stA(std::integral_constant<int, S>{});
        const uint4 *cB = stB(std::integral_constant<int, S>{});
        const uint4 *oA = stA(std::integral_constant<int, S + 1>{});
        const uint4 *oB = stB(std::integral_constant<int, S + 1>{});
        uint4 *dA = stA(std::integral_constant<int, S>{});      // receives A of step kt+2
        uint4 *dB = stB(std::integral_constant<int, S + 1>{});  // receives B of step kt+1
        uint32_t next[4];  // rows of step kt+1
#pragma unroll
        for (int i = 0; i < 4; ++i) next[i] = rows[i];
        load_rows(kt + 2, rows);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < 3) {
                read_tr(cB, ks + 1, wn * WTN, fb[(ks + 1) & 1], FNc{});
                read_tr(cA, ks + 1, wm * WTM, fa[(ks + 1) & 1], FMc{});
            } else {
                read_tr(oB, 0, wn * WTN, fb[0], FNc{});
                read_tr(oA, 0, wm * WTM, fa[0], FMc{});
            }
            if (ks == 0) dma(rB, ldb2, nb2, dB, next);
            if (ks == 3) dma(rA, lda2, ma2, dA, rows);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
            // per two MFMAs: three fragment reads, and in sub-steps 0 and 3 one LDS-DMA load
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
                if (ks == 0 || ks == 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // LDS-DMA load
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 2) {
                __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (kt0 < kt1) {
        const int nlist = (kte - kt0 + 2) * BK;
        load_row_list<512>(idx + kt0 * BK, (kt1 - kt0) * BK, nlist, sIdx, tid);
        __syncthreads();
        // steps kt0 (both operands) and kt0+1 (A; its B is loaded in step kt0's sub-step 0)
        load_rows(kt0, rows);
        dma(rA, lda2, ma2, sA0, rows);
        dma(rB, ldb2, nb2, sB0, rows);
        load_rows(kt0 + 1, rows);
        dma(rA, lda2, ma2, sA1, rows);
        __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_tr(sB0, 0, wn * WTN, fb[0], FNc{});
        read_tr(sA0, 0, wm * WTM, fa[0], FMc{});
        for (int kt = kt0; kt < kte; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    uint4 *stage = ((w >> 1) == 0 ? sA0 : (w >> 1) == 1 ? sA1 : (w >> 1) == 2 ? sB0 : sB1) + (w & 1) * (BUF / 2);
    store_tile_w8<SPLIT>(g, acc, stage, m0, n0, b, split, wm, wn, lane);
}

// Reduced product with a narrow output (m <= 128) whose kept A columns are
// gathered inside the kernel: the token-axis product P[:, T] V[T, :] of an
// attention head (Sec. 3.2, "Attention"), where A = P is L_q x L_k, B = V is
// L_k x d_v and T is the kept token set.  With m = d_v = 128 the output is a
// thin strip, so packing A[:, I] (a k x n write and read) would cost more
// than the product; instead the kernel reads A once, in coalesced pieces.
//
// A workgroup of eight waves owns 256 rows of one batch entry (and one
// 128-column block of the output).  The kept list is split by 64-column
// windows of A; for each window holding at least one kept column, the
// 256 x 64 block of A (128-byte row pieces, 32 KB) and the window's kept
// rows of B (compacted, zero rows up to 64) are copied into one of three LDS
// stages by LDS-DMA buffer loads, two windows ahead, so that 64 KB of A per
// CU is in flight.  Each wave multiplies its 32 rows: the A fragments are
// gathered from the staged block at the kept positions (one 8-byte LDS read
// of eight window offsets, then 16-bit reads; slots past the window's count
// read as zero), the B fragments are read with ds_read_b64_tr_b16, and four
// 32x32 column blocks accumulate in fp32 over the kept columns in ascending
// order.  Windows without kept columns are never read.
//
// Set-up: the list is copied into LDS (over the third A stage, free until
// the first refill), each window's first entry is found by binary search,
// the non-empty windows are compacted in order and every entry's offset
// within its window is stored as a byte at [window][rank], the form the
// gather reads.  Layouts: staged A row r holds its eight 16-byte chunks at
// c ^ (r & 7); staged B row k at c ^ 2(k & 3) (16 chunks of 8 columns).
// Every thread issues exactly six LDS-DMA loads per window (four of A, two
// of B; rows past n, past the window's count or of padding windows read as
// zero), so "window e landed" is vmcnt(6) while window e+1 is in flight.
// One barrier per window publishes its stage and certifies that the stage
// refilled next (read for the previous window) is no longer read.
// Workgroups are dealt to XCDs in contiguous runs of row blocks of one batch
// entry, so the entries sharing one B (grouped-query attention) read its
// rows from the same L2.
constexpr int kGcolWindows = (int)(kGcolMaxD / 64);

template <int S>
__device__ __forceinline__ uint4 *gcol_stage(uint4 *a0, uint4 *a1, uint4 *a2) {
    if constexpr (S % 3 == 0) return a0;
    else if constexpr (S % 3 == 1) return a1;
    else return a2;
}

__global__ __launch_bounds__(512, 1) void gemm_gcol_kernel(GemmArgs g) {
    constexpr int NW = 8, NT = NW * 64;
    constexpr int BM = 32 * NW, BN = 128, W = 64;
    constexpr int PCH = W / 8;      // 16-byte chunks per staged A row
    constexpr int VCH = BN / 8;     // 16-byte chunks per staged B row
    constexpr int PBUF = BM * PCH;  // uint4 per A stage (32 KB)
    constexpr int VBUF = W * VCH;   // uint4 per B stage (16 KB)
    constexpr int MAXWIN = kGcolWindows;
    static_assert(kGcolMaxD * 2 <= PBUF * 16, "the list must fit in one A stage");
    static_assert(MAXWIN < NT, "one thread per window");
    __shared__ uint4 sP0[PBUF];
    __shared__ uint4 sP1[PBUF];
    __shared__ uint4 sP2[PBUF];
    __shared__ uint4 sV0[VBUF];
    __shared__ uint4 sV1[VBUF];
    __shared__ uint4 sV2[VBUF];
    __shared__ __align__(16) uint8_t sPos[MAXWIN * W];  // offsets of window u's kept columns, by rank
    __shared__ uint16_t sStart[MAXWIN + 1];              // first list entry at or past column 64u
    __shared__ uint16_t sWin[MAXWIN + 4];                // windows holding kept columns (+ padding)
    __shared__ uint16_t sBeg[MAXWIN + 4];                // their first list entries (+ the end)
    __shared__ int sCnt[NW];
    typedef __attribute__((address_space(3))) void lds_t;
    uint16_t *sIdx = reinterpret_cast<uint16_t *>(sP2);  // the list, during set-up only

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int tiles_m = (int)((g.n + BM - 1) / BM), tiles_n = (int)((g.m + BN - 1) / BN);
    const int T = tiles_m * tiles_n * (int)g.batch;
    int t = blockIdx.x;
    if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
    const int64_t b = t / (tiles_m * tiles_n);
    const int rem = t - (int)b * tiles_m * tiles_n;
    const int tm = rem % tiles_m, tn = rem / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + b * g.strideA, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (b / g.group) * g.strideB, g.b_bytes);
    const int32_t *idx = g.idx + b * g.ld_idx;
    const int k = (int)g.k;
    const uint32_t lda2 = (uint32_t)(g.lda * 2), ldb2 = (uint32_t)(g.ldb * 2);

    // set-up (entries -1 read as 0xffff, above every column)
    load_row_list<NT>(idx, k, k, sIdx, tid);
    __syncthreads();
    if (tid <= MAXWIN) {
        int lo = 0, hi = k;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if ((int)sIdx[mid] < tid * W) lo = mid + 1; else hi = mid;
        }
        sStart[tid] = (uint16_t)lo;
    }
    __syncthreads();
    const bool ne = tid < MAXWIN && sStart[tid + 1] > sStart[tid];
    const uint64_t bal = __ballot(ne);
    if (lane == 0) sCnt[w] = __popcll(bal);
    for (int j = tid; j < k; j += NT) {
        const int v = sIdx[j];
        if (v < MAXWIN * W) sPos[(v >> 6) * W + j - sStart[v >> 6]] = (uint8_t)(v & (W - 1));
    }
    __syncthreads();
    int off = 0, nwin = 0;
    for (int i = 0; i < NW; ++i) {
        off += i < w ? sCnt[i] : 0;
        nwin += sCnt[i];
    }
    if (ne) {
        const int pos = off + __popcll(bal & ((1ull << lane) - 1ull));
        sWin[pos] = (uint16_t)tid;
        sBeg[pos] = sStart[tid];
    }
    // up to two empty windows pad the count to a multiple of three (the
    // unrolled stage rotation); they load zeros and multiply nothing, and
    // index npad stands for the refills past the end
    const int npad = (nwin + 2) / 3 * 3;
    if (tid >= nwin && tid <= npad + 1) {
        sWin[tid] = 0;
        sBeg[tid] = sStart[MAXWIN];
    }
    __syncthreads();

    // loads of window e: rows 32w + 8q + lane/8 of A (chunk lane%8 of the
    // stage row), kept rows 8w + 4q + lane/16 of B
    auto issue = [&](int e, uint4 *dP, uint4 *dV) {
        const bool real = e < nwin;
        const int u = sWin[e], beg = sBeg[e], cnt = (int)sBeg[e + 1] - beg;  // padding: cnt = 0
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 32 * w + 8 * q + (lane >> 3);
            const uint32_t c = (uint32_t)((lane & 7) ^ (r & 7));
            const uint32_t o =
                real && m0 + r < g.n ? (uint32_t)((m0 + r) * lda2 + (uint32_t)(u * W) * 2u + c * 16u) : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_t *)&dP[(32 * w + 8 * q) * PCH], 16, o, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int kk = 8 * w + 4 * q + (lane >> 4);
            const uint32_t c = (uint32_t)((lane & 15) ^ ((kk & 3) << 1));
            const int64_t col = n0 + 8 * c;
            const uint32_t row = (uint32_t)(u * W + sPos[u * W + (kk & (W - 1))]);
            const uint32_t o = kk < cnt && col < g.m ? row * ldb2 + (uint32_t)col * 2u : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_t *)&dV[(8 * w + 4 * q) * VCH], 16, o, 0, 0, 0);
        }
    };

    f32x16_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    const int ar = 32 * w + (lane & 31);  // this lane's staged A row
    const int hsel = lane >> 5;
    // column p of staged row ar sits at byte ((p >> 3) ^ (ar & 7)) * 16 + (p & 7) * 2 of the row,
    // which is 2p ^ rsw: the swizzle only flips bits 4-6
    const uint32_t rsw = (uint32_t)(ar & 7) << 4;
    auto compute = [&](int e, const uint4 *cP, const uint4 *cV) __attribute__((always_inline)) {
        const int u = sWin[e], cnt = (int)sBeg[e + 1] - (int)sBeg[e];
        const char *prow = reinterpret_cast<const char *>(cP) + ar * (PCH * 16);
        // one k16 step; only a window's last, partial step masks slots past its count
        auto kstep = [&](int ks, auto Mc) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(Mc)::value;
            const uint2 pp = *reinterpret_cast<const uint2 *>(sPos + u * W + ks * 16 + hsel * 8);
            uint32_t pk[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t word = h < 2 ? pp.x : pp.y;
                uint32_t v2[2];
#pragma unroll
                for (int z = 0; z < 2; ++z) {
                    const uint32_t p = (word >> (8 * (2 * (h & 1) + z))) & (W - 1);
                    const uint32_t x = *reinterpret_cast<const uint16_t *>(prow + ((p << 1) ^ rsw));
                    v2[z] = !MASK || ks * 16 + hsel * 8 + 2 * h + z < cnt ? x : 0u;
                }
                pk[h] = v2[0] | (v2[1] << 16);
            }
            const bf16x8_t fa = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
            const int gq = lane >> 4, li = lane & 15;
            const int kbase = ks * 16 + 8 * (gq >> 1) + (li >> 2);
#pragma unroll
            for (int jn = 0; jn < 4; ++jn) {
                const int nn = jn * 32 + 16 * (gq & 1) + 4 * (li & 3);
                union {
                    v4i16_t h[2];
                    bf16x8_t v;
                } fb;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = kbase + 4 * hh;
                    const char *pb = reinterpret_cast<const char *>(&cV[kr * VCH + ((nn >> 3) ^ ((kr & 3) << 1))]) +
                                     ((nn >> 2) & 1) * 8;
                    fb.h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)pb);
                }
                // operands swapped: lane l holds output row l % 32
                acc[jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb.v, fa, acc[jn], 0, 0, 0);
            }
        };
        int ks = 0;
        for (; (ks + 1) * 16 <= cnt; ++ks) kstep(ks, std::false_type{});
        if (ks * 16 < cnt) kstep(ks, std::true_type{});
    };

    // window e: its loads landed once only window e+1's six are younger
    auto window = [&](int e, auto Sc) {
        constexpr int S = decltype(Sc)::value;
        __builtin_amdgcn_s_waitcnt(0x0f76);  // vmcnt(6)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(min(e + 2, npad), gcol_stage<S + 2>(sP0, sP1, sP2), gcol_stage<S + 2>(sV0, sV1, sV2));
        compute(e, gcol_stage<S>(sP0, sP1, sP2), gcol_stage<S>(sV0, sV1, sV2));
    };

    if (npad > 0) {
        issue(0, sP0, sV0);
        issue(1, sP1, sV1);
        for (int e = 0; e < npad; e += 3) {
            window(e, std::integral_constant<int, 0>{});
            window(e + 1, std::integral_constant<int, 1>{});
            window(e + 2, std::integral_constant<int, 2>{});
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load outlives the workgroup

    // lane l: row 32w + l % 32, columns 32 jn + 8 q + 4 (l / 32) + 0..3
    const int64_t row = m0 + ar;
    if (row < g.n) {
        uint16_t *yrow = g.Y + b * g.strideY + row * g.ldy;
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t col = n0 + jn * 32 + q * 8 + hsel * 4;
                if (col >= g.m) continue;  // m % 8 == 0: the four columns are all in or all out
                const uint32_t lo = pack_bf16x2(g.alpha * acc[jn][4 * q], g.alpha * acc[jn][4 * q + 1]);
                const uint32_t hi = pack_bf16x2(g.alpha * acc[jn][4 * q + 2], g.alpha * acc[jn][4 * q + 3]);
                *reinterpret_cast<uint2 *>(yrow + col) = make_uint2(lo, hi);
            }
    }
}

// Reduced product for one or two 64-entry K steps (kpad = 64 or 128), both
// operands in MFMA operand blocks (A: rows of A[:, I]; B: rows of B^T[:, I],
// i.e. the kept columns of the keys for Q K^T).  Such products are bound by
// writing Y (62 or 124 flop per output byte), so the kernel is persistent and
// built to keep the store stream at HBM speed.  A workgroup owns column
// strips (one batch entry, 512 columns) and walks down them in 64-row tiles.
// Its four waves (one per SIMD) each compute 64 rows x 128 columns of a
// tile, keep their strip's B fragments (KS = kpad / 16 sub-steps x 4 column
// blocks) in registers for the whole strip and load only the tile's A
// fragments per tile, right after the MFMAs that consumed the previous ones.
// A wave rounds its results to bf16, stages them in one of two LDS tile
// buffers and, after the workgroup barrier, stores 16 whole tile rows, one
// 1 KB row segment per store instruction; the stores drain while the next
// tile's MFMAs run.  1 KB row segments are the store pattern HBM absorbs
// fastest on MI355X (6.3 TB/s measured for runs of 64 x 1 KB tiles, against
// 5.3 TB/s for 256-byte segments).  Two stage buffers make one barrier per
// tile enough: a buffer is rewritten only after the barrier that follows
// every wave's reads of it.  Strips are dealt to workgroups in contiguous
// runs and runs to XCDs in order, so the strips of a batch entry share an
// XCD and its L2 copy of A.  Stage layout: 64 rows of 64 16-byte chunks,
// rows 65 chunks apart (the pad chunk spreads a column's rows over the LDS
// banks and keeps every staging address a lane base plus a constant).
constexpr int kStreamBM = 64, kStreamBN = 512;

template <int KS>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(GemmArgs g) {
    constexpr int BM = kStreamBM, BN = kStreamBN, WTN = 128, FM = 2, FN = 4, CPR = BN / 8 + 1;
    __shared__ uint4 stageL[2][BM * CPR];  // 2 x 65 KB
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t tiles_m = (g.n + BM - 1) / BM, tiles_n = (g.m + BN - 1) / BN;
    const int64_t strips = tiles_n * g.batch;
    const int G = gridDim.x;
    const int chunk = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int64_t per = (strips + G - 1) / G;
    const int64_t s0 = chunk * per, s1 = min(strips, s0 + per);
    const int count = s1 > s0 ? (int)((s1 - s0) * tiles_m) : 0;  // tiles of this workgroup
    const int tiles_n32 = (int)tiles_n, tiles_m32 = (int)tiles_m, s032 = (int)s0;
    auto coords = [&](int q, int &b, int &tm, int &tn) {
        const int qs = q / tiles_m32;
        const int s = s032 + qs;
        tm = q - qs * tiles_m32;
        b = s / tiles_n32;
        tn = s - b * tiles_n32;
    };

    bf16x8_t fa[KS][FM], fb[KS][FN];
    auto load_a = [&](int q) {
        int b, tm, tn;
        coords(q, b, tm, tn);
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + (int64_t)b * g.strideA, g.a_bytes);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t rb = (int64_t)tm * (BM / 32) + i;
            const uint32_t off = rb * 32 < g.n ? (uint32_t)(rb * KS * 1024 + lane * 16) : kOob;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) fa[ks][i] = as_bf16x8(buf_load16(rA, off + ks * 1024));
        }
    };
    auto load_b = [&](int q) {
        int b, tm, tn;
        coords(q, b, tm, tn);
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (int64_t)b * g.strideB, g.b_bytes);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t cb = (int64_t)tn * (BN / 32) + w * (WTN / 32) + j;
            const uint32_t off = cb * 32 < g.m ? (uint32_t)(cb * KS * 1024 + lane * 16) : kOob;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) fb[ks][j] = as_bf16x8(buf_load16(rB, off + ks * 1024));
        }
    };

    if (count > 0) {
        load_a(0);
        load_b(0);
    }
    // staging base of this lane's 8-byte pieces: row l%32 (+ 32 i), wave's 8 chunks, half l/32
    const int sbase = ((lane & 31) * CPR + w * (WTN / 8)) * 16 + (lane >> 5) * 8;
    for (int q = 0; q < count; ++q) {
        f32x16_t acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
        uint2 pk[FM][FN][4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    pk[i][j][qq] = make_uint2(pack_bf16x2(g.alpha * acc[i][j][4 * qq], g.alpha * acc[i][j][4 * qq + 1]),
                                              pack_bf16x2(g.alpha * acc[i][j][4 * qq + 2], g.alpha * acc[i][j][4 * qq + 3]));
        if (q + 1 < count) {
            if ((q + 1) % tiles_m32 == 0) load_b(q + 1);  // next strip
            load_a(q + 1);
        }
        // lane l, registers 4qq..4qq+3 of block (i, j): row i*32 + l%32,
        // columns j*32 + 8qq + 4(l/32) + 0..3 of this wave's 128 columns
        char *st = reinterpret_cast<char *>(stageL[q & 1]) + sbase;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    *reinterpret_cast<uint2 *>(st + (i * 32 * CPR + j * 4 + qq) * 16) = pk[i][j][qq];
        __syncthreads();
        // wave w stores tile rows 16 w .. 16 w + 15, one 1 KB row segment per instruction
        int b, tm, tn;
        coords(q, b, tm, tn);
        const int64_t m0 = (int64_t)tm * BM, col = (int64_t)tn * BN + lane * 8;
        const uint4 *stg = stageL[q & 1];
        uint16_t *Yb = g.Y + (int64_t)b * g.strideY;
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int r = w * 16 + it;
            const uint4 v = stg[r * CPR + lane];
            const int64_t row = m0 + r;
            if (row < g.n && col < g.m) *reinterpret_cast<uint4 *>(Yb + row * g.ldy + col) = v;
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
    int sp = 0;
    // eight partial rows in flight, still added in ascending split order
    for (; sp + 8 <= splits; sp += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4 *>(part + (int64_t)(sp + u) * total + q);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            s.x += v[u].x;
            s.y += v[u].y;
            s.z += v[u].z;
            s.w += v[u].w;
        }
    }
    for (; sp < splits; ++sp) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)sp * total + q);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    uint16_t *y = Y + b * strideY + row * ldy + col;
    uint32_t lo = pack_bf16x2(alpha * s.x, alpha * s.y);
    uint32_t hi = pack_bf16x2(alpha * s.z, alpha * s.w);
    *reinterpret_cast<uint2 *>(y) = make_uint2(lo, hi);
}

// Same sum for many splits: 64 four-column groups x 4 split groups per
// workgroup; split group g adds splits g, g+4, g+8, ... (ascending) with all
// its loads in flight, then the four group sums are added in the order
// 0, 1, 2, 3 (a fixed order, so results are bit-reproducible).
__global__ __launch_bounds__(256) void splitk_reduce_wide_kernel(const float *__restrict__ part, int splits, int64_t n,
                                                                 int64_t m, int64_t batch, float alpha,
                                                                 uint16_t *__restrict__ Y, int64_t ldy,
                                                                 int64_t strideY) {
    __shared__ float4 red[4][64];
    const int cq = threadIdx.x & 63, sg = threadIdx.x >> 6;
    const int64_t q = ((int64_t)blockIdx.x * 64 + cq) * 4;
    const int64_t plane = n * m;
    const int64_t total = plane * batch;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q < total) {
        int sp = sg;
        for (; sp + 12 < splits; sp += 16) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4 *>(part + (int64_t)(sp + 4 * u) * total + q);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
        }
        for (; sp < splits; sp += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)sp * total + q);
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
    }
    red[sg][cq] = s;
    __syncthreads();
    if (sg != 0 || q >= total) return;
    float4 t = red[0][cq];
#pragma unroll
    for (int g = 1; g < 4; ++g) {
        t.x += red[g][cq].x;
        t.y += red[g][cq].y;
        t.z += red[g][cq].z;
        t.w += red[g][cq].w;
    }
    const int64_t b = q / plane;
    const int64_t rc = q - b * plane;
    const int64_t row = rc / m, col = rc - row * m;
    uint16_t *y = Y + b * strideY + row * ldy + col;
    *reinterpret_cast<uint2 *>(y) = make_uint2(pack_bf16x2(alpha * t.x, alpha * t.y), pack_bf16x2(alpha * t.z, alpha * t.w));
}

// ------------------------------------------------------------------ pack
// dst[b][r][t] = src[b/group][r][idx[b][t]] for t < kpad, 0 where idx is -1
// (the padded index list is -1 beyond k).  Whole source rows are staged in
// LDS with 16-byte loads when `rows_per_wg` rows fit; each thread then reads
// the eight indices of one output chunk once and gathers that chunk for every
// staged row.  Without LDS staging the gathers read global memory.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ src, int64_t rows, int64_t d,
                                                   int64_t ld_src, int64_t src_stride, int64_t group,
                                                   const int32_t *__restrict__ idx_all, int64_t ld_idx,
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
    // separate LDS and global reads (use_lds is uniform): one pointer that
    // could be either would make every read a flat load
    auto gather = [&](int rr, const int32_t (&j)[8]) {
        uint32_t h[8];
        if (use_lds) {
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = j[e] >= 0 ? (uint32_t)rowbuf[rr * d + j[e]] : 0u;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = j[e] >= 0 ? (uint32_t)S[(r0 + rr) * ld_src + j[e]] : 0u;
        }
        return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    };
    for (int64_t c = tid; c < cpr; c += 256) {
        const int4 p0 = *reinterpret_cast<const int4 *>(idx + c * 8);
        const int4 p1 = *reinterpret_cast<const int4 *>(idx + c * 8 + 4);
        const int32_t j[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        for (int rr = 0; rr < nr; ++rr) *reinterpret_cast<uint4 *>(D + (r0 + rr) * kpad + c * 8) = gather(rr, j);
    }
}

// Pack into MFMA operand blocks (layout 1).  The output of one 32-row block
// and TT consecutive kept entries (a "tile": TT/16 operand blocks) is 2*TT
// bytes per row, written contiguously (each wave stores whole 1 KB blocks).
// Kept entries ascend, so a tile's source columns lie in the window
// [first entry, last valid entry + 1) of its 32 rows.  A workgroup owns one
// row block and a run of consecutive tiles and streams through them: while
// it gathers tile i out of one LDS window buffer and writes it, the 16-byte
// loads of tile i+1's window (and its index pieces) are already in flight
// into registers, then land in the other buffer.  Loads are issued before
// the stores of the same iteration, so waiting for them never waits for the
// stores.  A tile whose window is wider than the buffer (kPackWinChunks
// 16-byte chunks), or any tile when rows are not 16-byte aligned, gathers
// straight from memory instead.  Rows past `rows` and padding entries
// (index -1) are written as zero.
constexpr int kPackWinChunks = 40;                      // window capacity: 320 source columns
constexpr int kPackRowStride = kPackWinChunks * 8 + 8;  // u16 per staged row (16-byte pad)
constexpr int kPackMaxTiles = 64;                       // tiles per workgroup

template <int TT>
__global__ __launch_bounds__(256) void pack_blocks_kernel(const uint16_t *__restrict__ src, int64_t rows, int64_t d,
                                                          int64_t ld_src, int64_t src_stride, int64_t group,
                                                          const int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                          int64_t kpad, uint16_t *__restrict__ dst,
                                                          int64_t dst_stride, int vec_ok, int tiles_per_wg) {
    constexpr int PP = TT / 64;                        // output pieces per thread per tile
    constexpr int WPT = (32 * kPackWinChunks + 255) / 256;  // window chunks per thread
    __shared__ uint16_t win[2][32 * kPackRowStride];
    __shared__ int32_t span_lo[kPackMaxTiles], span_hi[kPackMaxTiles];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t rb = blockIdx.x, b = blockIdx.z;
    const int ntiles_all = (int)(kpad / TT);
    const int tt0 = (int)blockIdx.y * tiles_per_wg;
    const int nt = min(tiles_per_wg, ntiles_all - tt0);
    if (nt <= 0) return;
    const uint16_t *S = src + (b / group) * src_stride;
    const int32_t *idx = idx_all + b * ld_idx;
    uint16_t *D = dst + b * dst_stride;
    const int row = lane & 31;  // row within the block owned by this lane
    const int64_t grow = rb * 32 + row;
    const bool row_ok = grow < rows;
    const int nrows = (int)max((int64_t)0, min((int64_t)32, rows - rb * 32));

    // source span of every tile of this run: [first entry, last valid + 1)
    for (int q = tid; q < nt; q += 256) {
        const int64_t t0 = (int64_t)(tt0 + q) * TT;
        const int32_t lo = idx[t0];
        int32_t last = idx[t0 + TT - 1];
        if (last < 0 && lo >= 0) {
            int a = 0, z = TT - 1;
            while (a < z) {
                const int mid = (a + z + 1) >> 1;
                if (idx[t0 + mid] >= 0) a = mid; else z = mid - 1;
            }
            last = idx[t0 + a];
        }
        span_lo[q] = lo;
        span_hi[q] = lo >= 0 ? last + 1 : -1;
    }
    __syncthreads();

    auto fits = [&](int q) {
        const int32_t lo = span_lo[q];
        return vec_ok && lo >= 0 && (span_hi[q] - (lo & ~7) + 7) / 8 <= kPackWinChunks;
    };
    // 16-byte loads of tile q's window (rows x chunks); chunk c of row r
    // goes to register slot (r * chunks + c - tid) / 256
    auto load_window = [&](int q, uint4 (&wr)[WPT]) {
        if (!fits(q)) return;
        const int32_t w0 = span_lo[q] & ~7;
        const int chunks = (span_hi[q] - w0 + 7) / 8;  // d % 8 == 0: chunks stay inside the row
#pragma unroll
        for (int u = 0; u < WPT; ++u) {
            const int e = tid + u * 256;
            const int r = e / kPackWinChunks, c = e - r * kPackWinChunks;
            if (r < nrows && c < chunks)
                wr[u] = *reinterpret_cast<const uint4 *>(S + (rb * 32 + r) * ld_src + w0 + c * 8);
        }
    };
    auto store_window = [&](int q, const uint4 (&wr)[WPT], uint16_t *buf) {
        if (!fits(q)) return;
        const int chunks = (span_hi[q] - (span_lo[q] & ~7) + 7) / 8;
#pragma unroll
        for (int u = 0; u < WPT; ++u) {
            const int e = tid + u * 256;
            const int r = e / kPackWinChunks, c = e - r * kPackWinChunks;
            if (r < nrows && c < chunks) {
                uint16_t *o = buf + r * kPackRowStride + c * 8;
                *reinterpret_cast<uint2 *>(o) = make_uint2(wr[u].x, wr[u].y);
                *reinterpret_cast<uint2 *>(o + 4) = make_uint2(wr[u].z, wr[u].w);
            }
        }
    };
    // this thread's index pieces of tile q: block w + 4h, lane -> (row, chunk)
    auto load_j = [&](int q, int32_t (&j)[PP][8]) {
        const int64_t t0 = (int64_t)(tt0 + q) * TT;
#pragma unroll
        for (int h = 0; h < PP; ++h) {
            const int64_t c = 2 * (w + 4 * h) + (lane >> 5);
            const int4 p0 = *reinterpret_cast<const int4 *>(idx + t0 + c * 8);
            const int4 p1 = *reinterpret_cast<const int4 *>(idx + t0 + c * 8 + 4);
            j[h][0] = p0.x; j[h][1] = p0.y; j[h][2] = p0.z; j[h][3] = p0.w;
            j[h][4] = p1.x; j[h][5] = p1.y; j[h][6] = p1.z; j[h][7] = p1.w;
        }
    };

    uint4 wr[WPT];
    int32_t jc[PP][8], jn[PP][8];
    load_window(0, wr);
    load_j(0, jc);
    store_window(0, wr, win[0]);
    __syncthreads();
    for (int q = 0; q < nt; ++q) {
        if (q + 1 < nt) {
            load_window(q + 1, wr);
            load_j(q + 1, jn);
        }
        const uint16_t *buf = win[q & 1];
        const bool fast = fits(q);
        const int32_t w0 = span_lo[q] & ~7;
        uint32_t hv[PP][8];
        // two separate loops (fast is uniform): one pointer that could be
        // either LDS or global memory would make every read a flat load
        if (fast) {
            // branch-free: padding entries read a valid slot and are zeroed after
            const uint16_t *mine = buf + row * kPackRowStride - w0;
#pragma unroll
            for (int h = 0; h < PP; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int32_t jj = jc[h][e];
                    const uint32_t v = mine[jj >= 0 ? jj : w0];
                    hv[h][e] = (row_ok && jj >= 0) ? v : 0u;
                }
        } else {
#pragma unroll
            for (int h = 0; h < PP; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int32_t jj = jc[h][e];
                    hv[h][e] = (row_ok && jj >= 0) ? (uint32_t)S[grow * ld_src + jj] : 0u;
                }
            // rare path: let its loads land here, so the LDS reads of the fast
            // path never wait for outstanding loads (those of the next window)
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        }
        const int64_t t0 = (int64_t)(tt0 + q) * TT;
#pragma unroll
        for (int h = 0; h < PP; ++h) {
            const int64_t blk = rb * (kpad >> 4) + (t0 >> 4) + (w + 4 * h);
            *reinterpret_cast<uint4 *>(D + blk * 512 + lane * 8) =
                make_uint4(hv[h][0] | (hv[h][1] << 16), hv[h][2] | (hv[h][3] << 16), hv[h][4] | (hv[h][5] << 16),
                           hv[h][6] | (hv[h][7] << 16));
        }
        if (q + 1 < nt) {
            store_window(q + 1, wr, win[(q + 1) & 1]);
#pragma unroll
            for (int h = 0; h < PP; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) jc[h][e] = jn[h][e];
        }
        __syncthreads();
    }
}

// Pack of short rows (d <= 128: attention head dimensions) into MFMA
// operand blocks.  A workgroup takes 256 consecutive rows; its 256 threads
// read them with coalesced 16-byte loads (all issued up front) into LDS rows
// padded to an odd number of 8-byte words, then thread r gathers the kept
// entries of row r (the same columns for every row, so a wave's 64 reads of
// one entry hit 64 rows: at most two lanes per bank) and writes its 16-byte
// pieces; for one piece the 32 rows of a block are 512 contiguous bytes.
// Rows past `rows` and padding entries (index -1) are written as zero.
template <int D>
__global__ __launch_bounds__(256) void pack_short_rows_kernel(const uint16_t *__restrict__ src, int64_t rows,
                                                              int64_t ld_src, int64_t src_stride, int64_t group,
                                                              const int32_t *__restrict__ idx_all, int64_t ld_idx,
                                                              int64_t kpad, uint16_t *__restrict__ dst,
                                                              int64_t dst_stride) {
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int STRIDE = D / 4 + 1;    // 8-byte words per LDS row (odd)
    constexpr int PER = CPR;             // chunk loads per thread (256 rows x CPR chunks / 256)
    __shared__ uint2 rowl[256 * STRIDE];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * 256;
    const uint16_t *S = src + (b / group) * src_stride;
    const int32_t *idx = idx_all + b * ld_idx;
    uint16_t *Dp = dst + b * dst_stride;
    const int nr = (int)min((int64_t)256, rows - r0);

    uint4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * 256 + tid;  // chunk e: row e / CPR, chunk e % CPR
        const int r = e / CPR, c = e % CPR;
        v[u] = r < nr ? *reinterpret_cast<const uint4 *>(S + (r0 + r) * ld_src + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = u * 256 + tid;
        const int r = e / CPR, c = e % CPR;
        rowl[r * STRIDE + 2 * c] = make_uint2(v[u].x, v[u].y);
        rowl[r * STRIDE + 2 * c + 1] = make_uint2(v[u].z, v[u].w);
    }
    __syncthreads();
    const uint16_t *mine = reinterpret_cast<const uint16_t *>(rowl + tid * STRIDE);
    const int64_t row = r0 + tid;
    const int64_t blk = row >> 5;
    if (row >= ((rows + 31) & ~(int64_t)31)) return;  // past the last 32-row block of the output
    // eight kept columns per piece: their numbers in one scalar load, then
    // eight LDS reads issued together (padding entries read column 0 and are
    // replaced by zero), so no read waits on another
#pragma unroll 2
    for (int c = 0; c < (int)(kpad / 8); ++c) {
        int32_t j[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) j[e] = idx[c * 8 + e];  // uniform: scalar loads
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = mine[max(j[e], 0)];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (j[e] >= 0 && tid < nr) ? h[e] : 0u;
        *reinterpret_cast<uint4 *>(Dp + ((blk * (kpad >> 4) + (c >> 1)) * 64 + (c & 1) * 32 + (row & 31)) * 8) =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
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

static GemmConfig gemm_choose_tile(int64_t n, int64_t m, int64_t k, int64_t batch);

// The A-direct kernel needs row-major B (rows gathered through the list),
// kept row numbers below 0xffff and a per-split K range whose list fits its
// 64 KB of LDS (32768 entries).
static bool adirect_ok(int64_t kpad, int splits, int64_t d, int transB) {
    if (transB || d >= 0xffff) return false;
    const int64_t KT = kpad / BK;
    const int64_t per = ((KT + splits - 1) / splits + 1) & ~1LL;
    return per * BK <= 32768;
}

// The LDS-DMA variant has the same needs, keeps its list in 32 KB (the
// padded range plus two steps) and rounds each split's K steps up to a
// multiple of three.  Inside the whole pipeline (operands partly resident in
// the caches) its steps measured 1-2% faster on MI355X, so it is taken only
// where that rounding adds at most 2% of the steps.
static bool bdma_ok(int64_t kpad, int splits, int64_t d, int transB) {
    if (transB || d >= 0xffff) return false;
    const int64_t KT = kpad / BK;
    const int64_t per = std::min<int64_t>(((KT + splits - 1) / splits + 1) & ~1LL, KT);
    const int64_t per3 = (per + 2) / 3 * 3;
    return (per3 + 2) * BK <= kBdmaListRows && per3 * 100 <= per * 102;
}

// The two-operand LDS-DMA kernel keeps the list of a split's K range (plus
// the two steps loaded past it) in 16 KB.
static bool tdma_ok(int64_t kpad, int splits, int64_t d, int bq = 0) {
    if (d >= 0xffff) return false;
    const int64_t KT = kpad / BK;
    const int64_t per = std::min<int64_t>(((KT + splits - 1) / splits + 1) & ~1LL, KT);
    return (per + 2) * BK <= (bq ? kTdmaListRowsQ : kTdmaListRows);
}

bool gemm_tdma_fits(int64_t kpad, int splits, int64_t d, int bq) { return tdma_ok(kpad, splits, d, bq); }

GemmConfig gemm_choose_transposed(int64_t n, int64_t m, int64_t k, int64_t d) {
    GemmConfig c = gemm_choose_tile(n, m, k, 1);
    if (c.tile == 0 && tdma_ok((k + 127) / 128 * 128, c.splits, d))
        c.tile = 5;
    else
        c.tile = -1;
    return c;
}

GemmConfig gemm_choose(int64_t n, int64_t m, int64_t k, int64_t batch, int64_t d, int transB) {
    if (transB && k <= 2 * BK && ((n + 255) / 256) * ((m + 255) / 256) * batch >= 512) {
        // one or two K steps, many tiles (scores Q K^T): write-bound streaming kernel
        GemmConfig c;
        c.tile = 3;
        c.splits = 1;
        return c;
    }
    GemmConfig c = gemm_choose_tile(n, m, k, batch);
    const int64_t kpad = (k + 127) / 128 * 128;
    if (c.tile == 0 && bdma_ok(kpad, c.splits, d, transB))
        c.tile = 4;
    else if (c.tile == 0 && adirect_ok(kpad, c.splits, d, transB))
        c.tile = 2;
    return c;
}

static GemmConfig gemm_choose_tile(int64_t n, int64_t m, int64_t k, int64_t batch) {
    GemmConfig c;
    const int64_t big = ((n + 255) / 256) * ((m + 255) / 256) * batch;
    const int64_t ksteps = (k + BK - 1) / BK;
    if (ksteps <= 4) {
        // short contractions are bound by writing Y: 128x128 tiles (64 KB of
        // LDS) let two workgroups share a CU and overlap stores with MFMAs
        c.tile = 1;
        c.splits = 1;
        return c;
    }
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
    if (c.tile == 3) {
        if ((a.kpad != BK && a.kpad != 2 * BK) || a.splits != 1) return hipErrorInvalidValue;
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
        const int64_t strips = ((a.m + kStreamBN - 1) / kStreamBN) * a.batch;
        const unsigned grid = (unsigned)std::min<int64_t>(strips, (int64_t)cus);
        if (a.kpad == BK)
            gemm_stream_kernel<4><<<grid, 256, 0, stream>>>(a);
        else
            gemm_stream_kernel<8><<<grid, 256, 0, stream>>>(a);
        return hipGetLastError();
    }
    // the row-list kernels read their lists in 16-byte pieces
    const bool list_aligned = ((uintptr_t)a.idx & 15) == 0 && a.ld_idx % 4 == 0;
    if (c.tile == 5) {
        if (a.bmode != 0 || a.batch != 1 || !list_aligned || !tdma_ok(a.kpad, a.splits, 0, a.bq))
            return hipErrorInvalidValue;
        const int64_t tiles = ((a.n + 255) / 256) * ((a.m + 255) / 256);
        dim3 grid((unsigned)tiles, (unsigned)a.splits, 1);
        if (a.bq != 0) {
            // 8-bit B: rows of m codes (16-byte pieces), one fp32 scale per column
            if (a.epi != 0 || a.bq > 2 || !a.colscale || a.m % 16 || a.ldb % 16 || ((uintptr_t)a.colscale & 15))
                return hipErrorInvalidValue;
            if (a.bq == 1) {
                if (a.splits > 1)
                    gemm_tdma_kernel<true, 0, 1><<<grid, 256, 0, stream>>>(a);
                else
                    gemm_tdma_kernel<false, 0, 1><<<grid, 256, 0, stream>>>(a);
            } else {
                if (a.splits > 1)
                    gemm_tdma_kernel<true, 0, 2><<<grid, 256, 0, stream>>>(a);
                else
                    gemm_tdma_kernel<false, 0, 2><<<grid, 256, 0, stream>>>(a);
            }
        } else if (a.epi == 1) {
            // SwiGLU needs whole sums: one K range; the interleaved operand is 2 x (outputs) wide
            if (a.splits != 1 || a.m % 64 != 0 || (a.Y && a.ldy < a.m / 2) || (a.Yt && (!a.npart || a.n % 8)) ||
                (!a.Y && !a.Yt))
                return hipErrorInvalidValue;
            gemm_tdma_kernel<false, 1><<<grid, 256, 0, stream>>>(a);
        } else if (a.splits > 1) {
            gemm_tdma8_kernel<true><<<grid, 512, 0, stream>>>(a);
        } else {
            gemm_tdma8_kernel<false><<<grid, 512, 0, stream>>>(a);
        }
        return hipGetLastError();
    }
    if (c.tile == 6) {
        if (a.bmode != 0 || a.splits != 1 || a.k > kGcolMaxD || a.k < 1 || a.m % 8 || a.n < 1 || a.batch < 1 ||
            !list_aligned || a.ld_idx < (a.k + 3) / 4 * 4)
            return hipErrorInvalidValue;
        const int64_t T = ((a.n + 255) / 256) * ((a.m + 127) / 128) * a.batch;
        if (T > INT32_MAX) return hipErrorInvalidValue;
        gemm_gcol_kernel<<<(unsigned)T, 512, 0, stream>>>(a);
        return hipGetLastError();
    }
    if (c.tile == 2 || c.tile == 4) {
        if (a.bmode != 0 || !list_aligned) return hipErrorInvalidValue;
        if (c.tile == 4 && (!list_aligned || !bdma_ok(a.kpad, a.splits, 0, 0))) return hipErrorInvalidValue;
        const int64_t tiles = ((a.n + 255) / 256) * ((a.m + 255) / 256);
        dim3 grid((unsigned)tiles, (unsigned)a.splits, (unsigned)a.batch);
        if (c.tile == 4) {
            if (a.splits > 1)
                gemm_bdma_kernel<true><<<grid, 256, 0, stream>>>(a);
            else
                gemm_bdma_kernel<false><<<grid, 256, 0, stream>>>(a);
        } else if (a.splits > 1) {
            gemm_adirect_kernel<true><<<grid, 256, 0, stream>>>(a);
        } else {
            gemm_adirect_kernel<false><<<grid, 256, 0, stream>>>(a);
        }
        return hipGetLastError();
    }
    if (c.tile == 0) return launch_tile<256, 256, 2, 2>(a, stream);
    return launch_tile<128, 128, 2, 2>(a, stream);
}

namespace {
// One thread per 16-byte piece (8 outputs) of a row of the interleaved operand.
__global__ __launch_bounds__(256) void gated_weights_kernel(const uint16_t *__restrict__ Wg,
                                                            const uint16_t *__restrict__ Wu, int64_t d, int64_t m,
                                                            int transposed, uint16_t *__restrict__ Wgu) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // piece index
    const int64_t per_row = 2 * m / 8;
    if (q >= d * per_row) return;
    const int64_t row = q / per_row, oc = (q - row * per_row) * 8;
    const int64_t blk = oc / 64, within = oc % 64;
    const uint16_t *W = within < 32 ? Wg : Wu;
    const int64_t c = blk * 32 + within % 32;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = transposed ? W[(c + e) * d + row] : W[row * m + c + e];
    *reinterpret_cast<uint4 *>(Wgu + row * 2 * m + oc) =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}
}  // namespace

hipError_t launch_gated_weights(const uint16_t *Wg, const uint16_t *Wu, int64_t d, int64_t m, int transposed,
                                uint16_t *Wgu, hipStream_t stream) {
    if (d < 1 || m < 32 || m % 32 || ((uintptr_t)Wgu & 15)) return hipErrorInvalidValue;
    const int64_t pieces = d * (2 * m / 8);
    gated_weights_kernel<<<(unsigned)((pieces + 255) / 256), 256, 0, stream>>>(Wg, Wu, d, m, transposed, Wgu);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *part, int splits, int64_t n, int64_t m, int64_t batch, float alpha,
                                uint16_t *Y, int64_t ldy, int64_t strideY, hipStream_t stream) {
    const int64_t quads = n * m * batch / 4;
    if (splits >= 16 && quads < (1 << 20)) {
        splitk_reduce_wide_kernel<<<(unsigned)((quads + 63) / 64), 256, 0, stream>>>(part, splits, n, m, batch, alpha,
                                                                                   Y, ldy, strideY);
        return hipGetLastError();
    }
    // small outputs (decode rows) use 64-thread workgroups to spread over more CUs
    const int bs = quads < 65536 ? 64 : 256;
    splitk_reduce_kernel<<<(unsigned)((quads + bs - 1) / bs), bs, 0, stream>>>(part, splits, n, m, batch, alpha, Y,
                                                                              ldy, strideY);
    return hipGetLastError();
}

// LDS budget for staged rows in pack_kernel.
static constexpr int64_t kPackLdsBytes = 64 * 1024;

hipError_t launch_pack(const void *src, rmm_dtype_t dt, int64_t rows, int64_t d, int64_t ld_src, int64_t src_stride,
                       int64_t group, const int32_t *idx, int64_t ld_idx, int64_t kpad, void *dst,
                       int64_t dst_stride, int64_t batch, int layout, hipStream_t stream) {
    if (dt != RMM_BF16) return hipErrorInvalidValue;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (dev < 32 && !(g_pack_attr_done & (1u << dev))) {
        hipError_t e = allow_big_lds(&pack_kernel);
        if (e != hipSuccess) return e;
        g_pack_attr_done |= 1u << dev;
    }
    if (layout != 0) {
        if (kpad % 64 != 0) return hipErrorInvalidValue;
        const int vec = ((uintptr_t)src % 16 == 0) && (ld_src % 8 == 0) && (d % 8 == 0) && (src_stride % 8 == 0);
        if (vec && (d == 64 || d == 128) && (uintptr_t)dst % 16 == 0) {
            // padded output rows: whole 32-row blocks, written by the 256-row workgroups
            dim3 grid((unsigned)((rows + 255) / 256), (unsigned)batch);
            if (d == 64)
                pack_short_rows_kernel<64><<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(src), rows, ld_src,
                                                                     src_stride, group, idx, ld_idx, kpad,
                                                                     static_cast<uint16_t *>(dst), dst_stride);
            else
                pack_short_rows_kernel<128><<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(src), rows, ld_src,
                                                                      src_stride, group, idx, ld_idx, kpad,
                                                                      static_cast<uint16_t *>(dst), dst_stride);
            return hipGetLastError();
        }
        const int tt = kpad % 128 == 0 ? 128 : 64;
        const int64_t ntiles = kpad / tt, rblocks = (rows + 31) / 32;
        // runs of consecutive tiles per workgroup: about 768 workgroups in all
        int64_t per = (ntiles * rblocks * batch + 767) / 768;
        per = std::max<int64_t>(1, std::min<int64_t>(per, kPackMaxTiles));
        if ((ntiles + per - 1) / per > 65535) per = std::min<int64_t>(kPackMaxTiles, (ntiles + 65534) / 65535);
        dim3 grid((unsigned)rblocks, (unsigned)((ntiles + per - 1) / per), (unsigned)batch);
        if (tt == 128)
            pack_blocks_kernel<128><<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(src), rows, d, ld_src,
                                                              src_stride, group, idx, ld_idx, kpad,
                                                              static_cast<uint16_t *>(dst), dst_stride, vec, (int)per);
        else
            pack_blocks_kernel<64><<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(src), rows, d, ld_src,
                                                             src_stride, group, idx, ld_idx, kpad,
                                                             static_cast<uint16_t *>(dst), dst_stride, vec, (int)per);
        return hipGetLastError();
    }
    const int64_t row_bytes = d * 2;
    int rpw = (int)(kPackLdsBytes / row_bytes);
    const int use_lds = rpw >= 1;
    if (rpw > 8) rpw = 8;
    if (rpw < 1) rpw = 4;
    const int vec_ok = use_lds && ((uintptr_t)src % 16 == 0) && (ld_src % 8 == 0) && (d % 8 == 0) &&
                       (src_stride % 8 == 0);
    const size_t lds = use_lds ? (size_t)rpw * (size_t)row_bytes : 0;
    dim3 grid((unsigned)((rows + rpw - 1) / rpw), (unsigned)batch);
    pack_kernel<<<grid, 256, lds, stream>>>(static_cast<const uint16_t *>(src), rows, d, ld_src, src_stride, group,
                                            idx, ld_idx, kpad, static_cast<uint16_t *>(dst), dst_stride, rpw,
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
