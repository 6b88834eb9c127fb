// Attention with reduced scores, softmax fused ("Reduced Matrix
// Multiplication: Input-Adaptive Matrix-Product Reduction for LLM
// Inference", Sec. 3.2, "Attention"): per query head h the feature scores
// are Q_h's column norms, I_h = TopK of them, and
//   O_h = softmax(alpha * Q_h[:, I_h] K_g[:, I_h]^T + M) V_g,
// alpha = 1/sqrt(d_h), M the optional causal mask, g the grouped-query
// key/value head of h.  The reduced scores never reach HBM: each workgroup
// keeps a running row reference and row sum (online softmax) while it walks
// the keys, so HBM sees Q_I, K_I and V once and O once.
//
// Inputs: Q as given (each lane gathers its row's kept columns once), K_I
// packed per query head in MFMA operand blocks (1 KB per 32 rows x 16 kept
// dims; rows padded to 32 with zeros, dims to kq = 64 or 128 with zeros), V
// row-major (L_k x 128 per key/value head).
//
// Workgroup: 128 queries of one head, four waves of 32.  Each wave keeps its
// Q fragments in registers for the whole key loop.  K operand blocks (2 kq/16
// KB per 64-key block, contiguous in the packed buffer) and V rows (16 KB,
// chunk c of row k at c ^ 2(k & 3)) are copied into LDS stages by LDS-DMA
// loads; every thread issues the same number of loads per block (past the
// end: zeros), so "this group landed" is a fixed vmcnt while the next group
// is in flight, and one barrier per block both publishes a stage and frees
// the one refilled next.
//
// Per block a wave computes S^T (64 keys x its 32 queries) with the keys as
// the MFMA's first operand, so lane l holds query l % 32 and sixteen keys per
// 32-key half: the row maximum and sum need one exchange with lane l ^ 32
// (v_permlane32_swap).  The probabilities, rounded to bf16, are already an
// MFMA operand (lane = query, eight keys per lane in a fixed order) for
// O^T += V_block^T P^T; the V fragments are read with ds_read_b64_tr_b16
// from the rows in that same key order.  O^T keeps lane = query too, so
// rescaling and the final division by the row sum are per-lane scalars.
// Exponentials are exp2(fma(s, alpha log2 e, -m)); the row sum adds the
// bf16 probabilities the value product uses (v_dot2c_f32_bf16 with ones).
//
// Lazy reference: m, the reference subtracted before exponentiating, moves
// only when a block's row maximum exceeds it by more than kSlack (log2
// units).  Softmax does not depend on the reference, every probability stays
// below 2^kSlack (bf16 and fp32 hold it with room to spare), and the running
// output is rescaled (64 multiplies per lane) only on such a move, which
// after the first blocks of a row is rare.
//
// kq = 64 (the pipelined kernel): K is staged two blocks ahead of V and the
// loop is skewed, so one block step of a wave issues the softmax of block
// e+1 (exponentials, conversions), the value product of block e (16 MFMAs)
// and the scores of block e+2 (8 MFMAs) with no dependence between them: the
// vector work of the softmax issues in the shadow of the matrix
// instructions of the same wave.  kq = 128 keeps the unskewed loop (scores,
// softmax, value product of one block per step) with two stages, so that two
// workgroups still share a CU.
#include "rmm_internal.h"

#include <type_traits>

namespace rmm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 abf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 abf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float af32x16_t;
typedef short av4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void attn_lds_t;

constexpr uint32_t kAttnOob = 0x80000000u;  // offsets of rows that must read as zero
constexpr float kSlack = 8.f;               // the reference trails the row maximum by at most this (log2 units)
constexpr int kKeyBlock = 64;               // keys per block
constexpr int kVChunks = 16;                // 16-byte chunks per V row (128 columns)

__device__ __forceinline__ abf16x8_t attn_bf16x8(uint4 v) {
    union {
        uint4 u;
        abf16x8_t b;
    } x;
    x.u = v;
    return x.b;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void *base, int64_t bytes) {
    const int32_t nrec = (int32_t)min(bytes, (int64_t)0x7fffffff);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nrec, 0x00020000);
}

// stage S of NS (2 or 3) LDS stages
template <int NS, int S>
__device__ __forceinline__ uint4 *attn_stage(uint4 *a0, uint4 *a1, uint4 *a2) {
    if constexpr (S % NS == 0) return a0;
    else if constexpr (S % NS == 1) return a1;
    else return a2;
}

// max over the lane pair (l, l ^ 32) that holds one query
__device__ __forceinline__ float attn_pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float attn_pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The query tiles of one workgroup: head h, tile qt0 and, when the causal
// tiles are paired, tile qt1 (else -1).  Paired, workgroup p of a head takes
// tiles qtiles-1-p (the longest key range) and p (the shortest), so that
// every workgroup walks about the same number of key blocks and the launch
// has no tail of long tiles started late.
struct AttnSlot {
    int h, qt0, qt1;
};

__host__ __device__ inline int attn_units(int Lq, int qrows, int pair) {
    const int qtiles = (Lq + qrows - 1) / qrows;
    return pair ? (qtiles + 1) / 2 : qtiles;
}

template <int NW>
__device__ __forceinline__ AttnSlot attn_slot(const AttnArgs &g) {
    AttnSlot sl;
    const int qtiles = (g.Lq + 32 * NW - 1) / (32 * NW);
    const int units = attn_units(g.Lq, 32 * NW, g.pair);
    const int t = blockIdx.x;
    int rank;  // position of the workgroup within its head, in dispatch order
    if ((g.H & 7) == 0) {
        // workgroups go to the eight XCDs in turn: XCD t % 8 takes heads [x H/8, (x+1) H/8)
        // (with grouped queries, heads that share K and V rows), and within an XCD the
        // workgroups go out rank by rank across its heads: under the causal mask the
        // long tiles start first
        const int hpx = g.H >> 3, u = t >> 3;
        sl.h = (t & 7) * hpx + u % hpx;
        rank = u / hpx;
    } else {
        sl.h = t / units;
        rank = t - sl.h * units;
    }
    if (!g.causal) {
        sl.qt0 = rank;
        sl.qt1 = -1;
    } else {
        sl.qt0 = qtiles - 1 - rank;  // a causal tile's keys grow with its position
        sl.qt1 = g.pair && rank != qtiles - 1 - rank ? rank : -1;
    }
    return sl;
}

// What every kernel needs about its tile: head, first query, this lane's query.
struct AttnTile {
    int h, q0, qi, off, lim, wfirst;
};

template <int NW>
__device__ __forceinline__ AttnTile attn_tile(const AttnArgs &g, int h, int qt, int w, int lane) {
    AttnTile a;
    a.h = h;
    a.q0 = qt * 32 * NW;
    a.qi = a.q0 + 32 * w + (lane & 31);  // this lane's query
    a.off = g.Lk - g.Lq;                 // queries are the last Lq positions
    a.lim = g.causal ? min(g.Lk - 1, a.qi + a.off) : g.Lk - 1;  // last key this query sees
    a.wfirst = a.q0 + 32 * w + a.off;    // last key the wave's first query sees (causal)
    return a;
}

// Q fragments of this lane's row, gathered through the kept-column list once per
// tile: slot (s, k) of lane group hsel is column idx[16 s + 8 hsel + k] (zero past
// k and for rows past Lq).  Branch-free, so that every index load and then every
// element load is in flight at once (the list rows are 256-byte aligned; a -1
// entry reads column 0 and is zeroed).
template <int KS>
__device__ __forceinline__ void attn_gather_q(const AttnArgs &g, const AttnTile &a, int hsel, abf16x8_t (&qf)[KS]) {
    const int4 *kid = reinterpret_cast<const int4 *>(g.idx + (int64_t)a.h * g.ld_idx + 8 * hsel);
    const uint16_t *qrow = g.Q + ((int64_t)a.h * g.Lq + min(a.qi, g.Lq - 1)) * g.dh;
    const bool row_ok = a.qi < g.Lq;
    int c[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int4 lo = kid[4 * s], hi = kid[4 * s + 1];
        c[s][0] = lo.x, c[s][1] = lo.y, c[s][2] = lo.z, c[s][3] = lo.w;
        c[s][4] = hi.x, c[s][5] = hi.y, c[s][6] = hi.z, c[s][7] = hi.w;
    }
    uint32_t v[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int k = 0; k < 8; ++k) v[s][k] = qrow[max(c[s][k], 0)];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v0 = row_ok && c[s][2 * i] >= 0 ? v[s][2 * i] : 0u;
            const uint32_t v1 = row_ok && c[s][2 * i + 1] >= 0 ? v[s][2 * i + 1] : 0u;
            pk[i] = v0 | (v1 << 16);
        }
        qf[s] = attn_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
}

// True when the block starting at key0 has keys some query of this wave must
// not see (past Lk, or past the causal diagonal): a wave-uniform test.
__device__ __forceinline__ bool attn_block_masked(const AttnArgs &g, const AttnTile &a, int key0) {
    return key0 + kKeyBlock > g.Lk || (g.causal && key0 + kKeyBlock - 1 > a.wfirst);
}

// False once the block starting at key0 lies past the causal limit of every
// query of this wave (it and all later blocks add nothing for the wave)
__device__ __forceinline__ bool attn_wave_live(const AttnArgs &g, const AttnTile &a, int key0) {
    return !g.causal || key0 <= a.wfirst + 31;
}

// Key blocks of the slot's tiles from query tile qt on (this tile's and, on
// the first pass, the paired tile's)
template <int NW>
__device__ __forceinline__ int attn_blocks(const AttnArgs &g, int qt) {
    const int kend = g.causal ? min(g.Lk, qt * 32 * NW + 32 * NW + (g.Lk - g.Lq)) : g.Lk;
    return (kend + kKeyBlock - 1) / kKeyBlock;
}

// Two workgroups share a CU and the hardware issues for the older one first:
// left alone, it finishes well before the younger one, which then runs by
// itself on a half-idle CU.  Each block step sets the waves' priority from the
// fraction of the slot's key blocks still to do (four levels), so the one
// that is behind is served first and the two finish together.  Scheduling
// only: the results do not change.
__device__ __forceinline__ void attn_priority(int remaining, int total) {
    const int level = 4 * remaining / (total + 1);
    if (level >= 3) __builtin_amdgcn_s_setprio(3);
    else if (level == 2) __builtin_amdgcn_s_setprio(2);
    else if (level == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// LDS-DMA copies of one group: the K operand blocks of key block kblk and the V
// rows of key block vblk (vblk < 0 or past the end: zeros), shared by the NW
// waves: attn_loads<KS, NW>() loads per thread, whatever the blocks.  The
// per-lane part of every copy offset is fixed (AttnCopies, computed once);
// a block adds a scalar, or kAttnOob when it is past the end or before the
// start.  Rows of the last V block past L_k lie past the buffer's end (V is
// L_k rows of 256 bytes), so they read as zero too.
template <int KS, int NW>
constexpr int attn_loads() {
    return 2 * KS / NW + 16 / NW;
}

template <int KS, int NW>
struct AttnCopies {
    static constexpr int KL = 2 * KS / NW;  // K operand blocks of 1 KB each wave copies per key block
    static constexpr int VL = 16 / NW;      // V copies of 1 KB (four rows) each wave makes per key block
    static_assert(KL * NW == 2 * KS && VL * NW == 16, "loads per wave");
    uint32_t k[KL], v[VL];

    __device__ __forceinline__ AttnCopies(uint32_t ldv2, int w, int lane) {
#pragma unroll
        for (int i = 0; i < KL; ++i) k[i] = (uint32_t)((w + NW * i) * 1024 + lane * 16);
#pragma unroll
        for (int q = 0; q < VL; ++q) {
            const int r = 4 * VL * w + 4 * q + (lane >> 4);
            v[q] = (uint32_t)r * ldv2 + (uint32_t)((lane & 15) ^ ((r & 3) << 1)) * 16u;
        }
    }

    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rK, __amdgpu_buffer_rsrc_t rV, uint32_t ldv2, int nblk,
                                          int w, int kblk, int vblk, uint4 *dK, uint4 *dV) const {
        const uint32_t kb = kblk < nblk ? (uint32_t)kblk * (uint32_t)(2 * KS * 1024) : kAttnOob;
        const uint32_t vb = vblk >= 0 && vblk < nblk ? (uint32_t)vblk * (uint32_t)kKeyBlock * ldv2 : kAttnOob;
#pragma unroll
        for (int i = 0; i < KL; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (attn_lds_t *)&dK[(w + NW * i) * 64], 16, k[i] + kb, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < VL; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (attn_lds_t *)&dV[(4 * VL * w + 4 * q) * kVChunks], 16,
                                                     v[q] + vb, 0, 0, 0);
    }
};

// S^T of one 64-key block for this wave's 32 queries: s[kb][r] is key
// 32 kb + 8 (r / 4) + 4 hsel + r % 4 of the block for query lane % 32
template <int KS>
__device__ __forceinline__ void attn_scores(const uint4 *cK, const abf16x8_t (&qf)[KS], int lane, af32x16_t (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
    for (int ss = 0; ss < KS; ++ss)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const abf16x8_t kf = attn_bf16x8(cK[(kb * KS + ss) * 64 + lane]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ss], s[kb], 0, 0, 0);
        }
}

// Drops the keys past lim from the scores of the block starting at key0.
// Online-softmax step for one 64-key block of this lane's query (scores s,
// masked keys at -inf): moves the reference m when the
// block's maximum clears it by more than kSlack, adds the block's
// probabilities to l and leaves them in bf16 as the value product's operand:
// pk[kb][st][i] packs slots 8 st + 2 i and 8 st + 2 i + 1 of half kb.
// Returns the factor the running output must be multiplied by (1: no move).
__device__ __forceinline__ void attn_mask(af32x16_t (&s)[2], int key0, int lim, int hsel) {
    // slot (kb, r) is key key0 + 4 hsel + 32 kb + 8 (r / 4) + r % 4: compare the
    // constant part with one per-lane bound (no per-slot key registers)
    const int rel = lim - key0 - 4 * hsel;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) > rel ? -INFINITY : s[kb][r];
}

__device__ __forceinline__ float attn_softmax(af32x16_t (&s)[2], float c, float &m, float &l,
                                              uint32_t (&pk)[2][2][4]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float mxs = attn_pair_max(mx) * c;  // c > 0: the scaled maximum
    float fac = 1.f;
    if (mxs > m + kSlack) {  // also the first finite block of a row (m = -inf): fac = 0
        fac = __builtin_amdgcn_exp2f(m - mxs);
        m = mxs;
    }
    // a row that has seen no finite score yet keeps m = -inf and gets only zeros
    const float nm = m == -INFINITY ? 0.f : -m;
    // raw v_exp_f32: arguments are <= kSlack, and results below 2^-126 (flushed to
    // zero) vanish against the probability of the row maximum (>= 1)
    const abf16x2_t ones = __builtin_bit_cast(abf16x2_t, 0x3f803f80u);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * st + 2 * i], c, nm));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * st + 2 * i + 1], c, nm));
                pk[kb][st][i] = pack_bf16x2(p0, p1);
                ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(abf16x2_t, pk[kb][st][i]), ones, ls, false);
            }
    l = l * fac + attn_pair_sum(ls);
    return fac;
}

// O^T += V^T P^T over one 64-key block: P slot k of lane group hsel in step
// (kb, st) is key 32 kb + 16 st + 8 (k / 4) + 4 hsel + k % 4 of the block, and
// the V fragments are read (transposed) from those rows
__device__ __forceinline__ void attn_pv(const uint4 *cV, const uint32_t (&pk)[2][2][4], int lane, af32x16_t (&o)[4]) {
    const int gq = lane >> 4, li = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const abf16x8_t pf =
                attn_bf16x8(make_uint4(pk[kb][st][0], pk[kb][st][1], pk[kb][st][2], pk[kb][st][3]));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nn = j * 32 + 16 * (gq & 1) + 4 * (li & 3);
                union {
                    av4i16_t hv[2];
                    abf16x8_t v;
                } vf;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = 32 * kb + 16 * st + 8 * hh + 4 * (gq >> 1) + (li >> 2);
                    const char *pb =
                        reinterpret_cast<const char *>(&cV[kr * kVChunks + ((nn >> 3) ^ ((kr & 3) << 1))]) +
                        ((nn >> 2) & 1) * 8;
                    vf.hv[hh] =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) av4i16_t *)pb);
                }
                o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.v, pf, o[j], 0, 0, 0);
            }
        }
}

__device__ __forceinline__ void attn_rescale(af32x16_t (&o)[4], float fac) {
    if (__ballot(fac != 1.f)) {  // some row's reference moved: rescale its running output
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[j][e] *= fac;
    }
}

// lane l: query qi, columns 32 j + 8 q + 4 hsel + 0..3
__device__ __forceinline__ void attn_store(const AttnArgs &g, const AttnTile &a, int hsel, const af32x16_t (&o)[4],
                                           float l) {
    if (a.qi >= g.Lq) return;
    const float inv = 1.f / l;
    uint16_t *orow = g.O + (int64_t)a.h * g.o_stride + (int64_t)a.qi * g.ldo;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = j * 32 + q * 8 + hsel * 4;
            const uint32_t lo = pack_bf16x2(o[j][4 * q] * inv, o[j][4 * q + 1] * inv);
            const uint32_t hi = pack_bf16x2(o[j][4 * q + 2] * inv, o[j][4 * q + 3] * inv);
            *reinterpret_cast<uint2 *>(orow + col) = make_uint2(lo, hi);
        }
}

// kq = 64.  Groups of loads: G_j = {K operand blocks of key block j + 2 into K
// stage (j + 2) % 3, V rows of key block j into V stage j % 3}, j >= -2 (V of
// j < 0: zeros).  Block step e waits for G_e (G_{e+1} stays in flight),
// passes the barrier, issues G_{e+2} into the stages read during step e - 1
// (K of block e + 1, V of block e - 1), then: softmax of block e + 1 (scores
// from step e - 1), value product of block e (P from step e - 1), scores of
// block e + 2.  NW waves (32 NW queries) share the stages, 72 KB of LDS.
template <int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_pipe_kernel(AttnArgs g) {
    constexpr int KS = 4;
    constexpr int KBUF = 2 * KS * 64;              // uint4 per K stage: 2 row groups x KS operand blocks of 1 KB
    constexpr int VBUF = kKeyBlock * kVChunks;     // uint4 per V stage (16 KB)
    constexpr int NL = attn_loads<KS, NW>();       // loads per thread per group
    static_assert(NL < 16, "vmcnt immediate");
    __shared__ uint4 sK0[KBUF];
    __shared__ uint4 sK1[KBUF];
    __shared__ uint4 sK2[KBUF];
    __shared__ uint4 sV0[VBUF];
    __shared__ uint4 sV1[VBUF];
    __shared__ uint4 sV2[VBUF];

    // the wave index from an SGPR: masking tests and LDS-DMA destinations stay scalar
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), hsel = lane >> 5;
    const AttnSlot sl = attn_slot<NW>(g);
    const __amdgpu_buffer_rsrc_t rK = attn_rsrc(g.K + (int64_t)sl.h * g.k_stride, g.k_bytes);
    const __amdgpu_buffer_rsrc_t rV = attn_rsrc(g.V + (int64_t)(sl.h / g.group) * g.v_stride, g.v_bytes);
    const uint32_t ldv2 = (uint32_t)(g.ldv * 2);
    const AttnCopies<KS, NW> cp(ldv2, w, lane);
    const float c = g.scale_log2;
    const int second = sl.qt1 >= 0 ? attn_blocks<NW>(g, sl.qt1) : 0;
    const int total = attn_blocks<NW>(g, sl.qt0) + second;
    for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? sl.qt0 : sl.qt1;
    if (qt < 0) break;
    if (pass) __syncthreads();  // the first tile's last reads of the stages are done
    const AttnTile a = attn_tile<NW>(g, sl.h, qt, w, lane);
    const int nblk = attn_blocks<NW>(g, qt);  // >= 1
    const int later = pass == 0 ? second : 0;  // blocks of the paired tile after this one

    auto issue = [&](int j, uint4 *dK, uint4 *dV) __attribute__((always_inline)) {
        cp.issue(rK, rV, ldv2, nblk, w, j + 2, j, dK, dV);
    };
    auto publish = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0f70 | NL);  // vmcnt(NL): only the newest group in flight
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    af32x16_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = 0.f;
    float m = -INFINITY, l = 0.f;
    af32x16_t s[2];
    uint32_t P[2][2][4];

    issue(-2, sK0, sV1);
    issue(-1, sK1, sV2);
    abf16x8_t qf[KS];  // gathered while the first copies are in flight
    attn_gather_q<KS>(g, a, hsel, qf);
    publish();  // G_-2: K of block 0
    issue(0, sK2, sV0);
    attn_scores<KS>(sK0, qf, lane, s);
    publish();  // G_-1: K of block 1
    issue(1, sK0, sV1);
    if (attn_block_masked(g, a, 0)) attn_mask(s, 0, a.lim, hsel);
    attn_softmax(s, c, m, l, P);
    attn_scores<KS>(sK1, qf, lane, s);

    auto block = [&](int e, auto Sc) __attribute__((always_inline)) {
        constexpr int S = decltype(Sc)::value;
        publish();  // G_e: V of block e, K of block e + 2
        attn_priority(nblk - e + later, total);
        if (!attn_wave_live(g, a, e * kKeyBlock)) {
            // past the causal limit of all of this wave's queries: blocks e and on add
            // nothing (every copy still goes out: the other waves read these stages)
            issue(e + 2, attn_stage<3, S + 1>(sK0, sK1, sK2), attn_stage<3, S + 2>(sV0, sV1, sV2));
            return;
        }
        // block e + 1 past the end is masked whole: its softmax changes nothing
        if (attn_block_masked(g, a, (e + 1) * kKeyBlock)) attn_mask(s, (e + 1) * kKeyBlock, a.lim, hsel);
        issue(e + 2, attn_stage<3, S + 1>(sK0, sK1, sK2), attn_stage<3, S + 2>(sV0, sV1, sV2));
        uint32_t Pn[2][2][4];
        const float fac = attn_softmax(s, c, m, l, Pn);
        attn_pv(attn_stage<3, S>(sV0, sV1, sV2), P, lane, o);
        // interleave: the transposed reads run four MFMAs ahead of the
        // value-product MFMA that uses them, the next group's copies go out one
        // per MFMA over the first six, and each MFMA is followed by a share of
        // the softmax's vector instructions
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if (i < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        // the new scores reuse the registers of the ones just consumed; none past
        // the last block (the masked softmax overwrites what s then holds)
        __builtin_amdgcn_sched_barrier(0);
        if (e + 2 < nblk) attn_scores<KS>(attn_stage<3, S + 2>(sK0, sK1, sK2), qf, lane, s);
        attn_rescale(o, fac);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int z = 0; z < 4; ++z) P[x][y][z] = Pn[x][y][z];
    };
    for (int e = 0;; e += 3) {
        block(e, std::integral_constant<int, 0>{});
        if (e + 1 >= nblk) break;
        block(e + 1, std::integral_constant<int, 1>{});
        if (e + 2 >= nblk) break;
        block(e + 2, std::integral_constant<int, 2>{});
        if (e + 3 >= nblk) break;
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load outlives the tile
    attn_store(g, a, hsel, o, l);
    }
}

// KS = kq / 16 = 8: two stages of 32 KB, one block ahead (64 KB), so that two
// workgroups share a CU; one block step does the scores, softmax and value
// product of one block.
template <int KS>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs g) {
    constexpr int NS = 2;
    constexpr int KBUF = 2 * KS * 64;
    constexpr int VBUF = kKeyBlock * kVChunks;
    __shared__ uint4 sK0[KBUF];
    __shared__ uint4 sK1[KBUF];
    __shared__ uint4 sV0[VBUF];
    __shared__ uint4 sV1[VBUF];

    // the wave index from an SGPR: masking tests and LDS-DMA destinations stay scalar
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), hsel = lane >> 5;
    const AttnSlot sl = attn_slot<4>(g);
    const __amdgpu_buffer_rsrc_t rK = attn_rsrc(g.K + (int64_t)sl.h * g.k_stride, g.k_bytes);
    const __amdgpu_buffer_rsrc_t rV = attn_rsrc(g.V + (int64_t)(sl.h / g.group) * g.v_stride, g.v_bytes);
    const uint32_t ldv2 = (uint32_t)(g.ldv * 2);
    const AttnCopies<KS, 4> cp(ldv2, w, lane);
    const float c = g.scale_log2;
    const int second = sl.qt1 >= 0 ? attn_blocks<4>(g, sl.qt1) : 0;
    const int total = attn_blocks<4>(g, sl.qt0) + second;
    for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? sl.qt0 : sl.qt1;
    if (qt < 0) break;
    if (pass) __syncthreads();  // the first tile's last reads of the stages are done
    const AttnTile a = attn_tile<4>(g, sl.h, qt, w, lane);
    const int nblk = attn_blocks<4>(g, qt);
    const int later = pass == 0 ? second : 0;  // blocks of the paired tile after this one
    const int npad = (nblk + NS - 1) / NS * NS;

    af32x16_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    abf16x8_t qf[KS];
    auto compute = [&](int blk, const uint4 *cK, const uint4 *cV) __attribute__((always_inline)) {
        if (blk >= nblk || !attn_wave_live(g, a, blk * kKeyBlock)) return;
        af32x16_t s[2];
        attn_scores<KS>(cK, qf, lane, s);
        uint32_t pk[2][2][4];
        if (attn_block_masked(g, a, blk * kKeyBlock)) attn_mask(s, blk * kKeyBlock, a.lim, hsel);
        const float fac = attn_softmax(s, c, m, l, pk);
        attn_rescale(o, fac);
        attn_pv(cV, pk, lane, o);
    };

    // block e+1 is issued only after the barrier, so wait for all
    auto block = [&](int e, auto Sc) __attribute__((always_inline)) {
        constexpr int S = decltype(Sc)::value;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        attn_priority(nblk - e + later, total);
        cp.issue(rK, rV, ldv2, nblk, w, min(e + 1, npad), min(e + 1, npad), attn_stage<NS, S + 1>(sK0, sK1, sK1),
                 attn_stage<NS, S + 1>(sV0, sV1, sV1));
        compute(e, attn_stage<NS, S>(sK0, sK1, sK1), attn_stage<NS, S>(sV0, sV1, sV1));
    };

    cp.issue(rK, rV, ldv2, nblk, w, 0, 0, sK0, sV0);
    attn_gather_q<KS>(g, a, hsel, qf);  // while the first copies are in flight
    for (int e = 0; e < npad; e += NS) {
        block(e, std::integral_constant<int, 0>{});
        block(e + 1, std::integral_constant<int, 1>{});
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load outlives the tile
    attn_store(g, a, hsel, o, l);
    }
}

}  // namespace

hipError_t launch_attention_fwd(const AttnArgs &a, int kq, hipStream_t stream) {
    if ((kq != 64 && kq != 128) || a.H < 1 || a.Lq < 1 || a.Lk < 1 || a.group < 1 || a.H % a.group ||
        (a.causal && a.Lq > a.Lk))
        return hipErrorInvalidValue;
    constexpr int kPipeWaves = 4;
    constexpr int qrows = 32 * kPipeWaves;  // queries per tile, both kernels
    // pair the causal tiles once there are more tiles than two workgroups per CU can hold
    AttnArgs b = a;
    b.pair = a.causal && (int64_t)((a.Lq + qrows - 1) / qrows) * a.H > 512;
    const int64_t T = (int64_t)attn_units(a.Lq, qrows, b.pair) * a.H;
    if (T > INT32_MAX) return hipErrorInvalidValue;
    if (kq == 64)
        attn_fwd_pipe_kernel<kPipeWaves><<<(unsigned)T, 64 * kPipeWaves, 0, stream>>>(b);
    else
        attn_fwd_kernel<8><<<(unsigned)T, 256, 0, stream>>>(b);
    return hipGetLastError();
}

}  // namespace rmm
