// Attention with reduced scores, softmax fused ("Reduced Matrix
// Multiplication: Input-Adaptive Matrix-Product Reduction for LLM
// Inference", Sec. 3.2, "Attention"): per query head h the feature scores
// are Q_h's column norms, I_h = TopK of them, and
//   O_h = softmax(alpha * Q_h[:, I_h] K_g[:, I_h]^T + M) V_g,
// alpha = 1/sqrt(d_h), M the optional causal mask, g the grouped-query
// key/value head of h.  The reduced scores never reach HBM: each workgroup
// keeps a running row maximum and row sum (online softmax) while it walks the
// keys, so HBM sees Q_I, K_I and V once and O once.
//
// Inputs: Q as given (each lane gathers its row's kept columns once), K_I
// packed per query head in MFMA operand blocks (1 KB per 32 rows x 16 kept
// dims; rows padded to 32 with zeros, dims to kq = 64 or 128 with zeros), V
// row-major (L_k x 128 per key/value head).
//
// Workgroup: 128 queries of one head, four waves of 32.  Each wave keeps its
// Q fragments in registers for the whole key loop.  Per 64-key block the K
// operand blocks (2 kq/16 KB, contiguous in the packed buffer) and the V rows
// (16 KB, chunk c of row k at c ^ 2(k & 3)) are copied into one of three LDS
// stages by LDS-DMA loads, two blocks ahead; every thread issues the same
// number of loads per block (past the end: zeros), so "block e landed" is a
// fixed vmcnt while block e+1 is in flight, and one barrier per block both
// publishes a stage and frees the one refilled next.
//
// Per block a wave computes S^T (64 keys x its 32 queries) with the keys as
// the MFMA's first operand, so lane l holds query l % 32 and sixteen keys per
// 32-key half: the row maximum and sum need one exchange with lane l ^ 32.
// The probabilities, rounded to bf16, are already an MFMA operand (lane =
// query, eight keys per lane in a fixed order) for O^T += V_block^T P^T; the
// V fragments are read with ds_read_b64_tr_b16 from the rows in that same key
// order.  O^T keeps lane = query too, so rescaling by exp(m_old - m_new) and
// the final division by the row sum are per-lane scalars.  Exponentials are
// exp2 of scores pre-scaled by alpha * log2(e).
#include "rmm_internal.h"

#include <type_traits>

namespace rmm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 abf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float af32x16_t;
typedef short av4i16_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kAttnOob = 0x80000000u;  // offsets of rows that must read as zero

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

// KS = kq / 16.  kq = 64: three stages, two blocks ahead (72 KB); kq = 128:
// two stages, one block ahead (64 KB), so that two workgroups share a CU in
// both cases.
template <int KS>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs g) {
    constexpr int NS = KS == 4 ? 3 : 2;   // LDS stages
    constexpr int KB = 64;                // keys per block
    constexpr int KBUF = 2 * KS * 64;     // uint4 per K stage: 2 row groups x KS operand blocks of 1 KB
    constexpr int VCH = 16;               // 16-byte chunks per V row (128 columns)
    constexpr int VBUF = KB * VCH;        // uint4 per V stage (16 KB)
    constexpr int KL = 2 * KS / 4;        // K operand blocks each wave copies per key block
    constexpr int NL = KL + 4;            // loads per thread per key block
    static_assert(NL < 16, "vmcnt immediate");
    __shared__ uint4 sK0[KBUF];
    __shared__ uint4 sK1[KBUF];
    __shared__ uint4 sK2[NS == 3 ? KBUF : 1];
    __shared__ uint4 sV0[VBUF];
    __shared__ uint4 sV1[VBUF];
    __shared__ uint4 sV2[NS == 3 ? VBUF : 1];
    typedef __attribute__((address_space(3))) void lds_t;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hsel = lane >> 5;
    const int qtiles = (g.Lq + 127) / 128;
    const int T = qtiles * g.H;
    int t = blockIdx.x;
    if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);  // each XCD takes a contiguous run of tiles
    const int h = t / qtiles;
    int qt = t - h * qtiles;
    if (g.causal) qt = qtiles - 1 - qt;  // a causal tile's keys grow with its position: longest first
    const int q0 = qt * 128;
    const int qi = q0 + 32 * w + (lane & 31);  // this lane's query
    const int off = g.Lk - g.Lq;                // queries are the last Lq positions

    const __amdgpu_buffer_rsrc_t rK = attn_rsrc(g.K + (int64_t)h * g.k_stride, g.k_bytes);
    const __amdgpu_buffer_rsrc_t rV = attn_rsrc(g.V + (int64_t)(h / g.group) * g.v_stride, g.v_bytes);
    const uint32_t ldv2 = (uint32_t)(g.ldv * 2);

    // Q fragments of this lane's row, gathered through the kept-column list once per
    // workgroup: slot (s, k) of lane group hsel is column idx[16 s + 8 hsel + k]
    // (zero past k and for rows past Lq)
    abf16x8_t qf[KS];
    {
        const int32_t *kid = g.idx + (int64_t)h * g.ld_idx + 8 * hsel;
        const uint16_t *qrow = g.Q + ((int64_t)h * g.Lq + min(qi, g.Lq - 1)) * g.dh;
        const bool row_ok = qi < g.Lq;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint32_t pk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c0 = kid[16 * s + 2 * i], c1 = kid[16 * s + 2 * i + 1];
                const uint32_t v0 = row_ok && c0 >= 0 ? qrow[c0] : 0u;
                const uint32_t v1 = row_ok && c1 >= 0 ? qrow[c1] : 0u;
                pk[i] = v0 | (v1 << 16);
            }
            qf[s] = attn_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }
    }

    const int kend = g.causal ? min(g.Lk, q0 + 128 + off) : g.Lk;
    const int nblk = (kend + KB - 1) / KB;
    const int npad = (nblk + NS - 1) / NS * NS;

    auto issue = [&](int blk, uint4 *dK, uint4 *dV) __attribute__((always_inline)) {
        const bool real = blk < nblk;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int b = w + 4 * i;  // operand block within the key block
            const uint32_t o = real ? (uint32_t)((blk * 2 * KS + b) * 1024 + lane * 16) : kAttnOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_t *)&dK[b * 64], 16, o, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 16 * w + 4 * q + (lane >> 4);
            const uint32_t c = (uint32_t)((lane & 15) ^ ((r & 3) << 1));
            const int key = blk * KB + r;
            const uint32_t o = real && key < g.Lk ? (uint32_t)key * ldv2 + c * 16u : kAttnOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_t *)&dV[(16 * w + 4 * q) * VCH], 16, o, 0, 0, 0);
        }
    };

    af32x16_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    auto compute = [&](int blk, const uint4 *cK, const uint4 *cV) __attribute__((always_inline)) {
        if (blk >= nblk) return;
        const int key0 = blk * KB;
        af32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
        for (int ss = 0; ss < KS; ++ss) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const abf16x8_t kf = attn_bf16x8(cK[(kb * KS + ss) * 64 + lane]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ss], s[kb], 0, 0, 0);
            }
        }
        // s[kb][r]: key key0 + 32 kb + 8 (r / 4) + 4 hsel + r % 4 for query qi; only blocks
        // reaching past Lk or past the wave's first query need the mask (a wave-uniform test)
        const bool masked = key0 + KB > g.Lk || (g.causal && key0 + KB - 1 > q0 + 32 * w + off);
        float mx = -INFINITY;
        if (masked) {
            const int lim = g.causal ? min(g.Lk - 1, qi + off) : g.Lk - 1;  // last key this query sees
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hsel + (r & 3);
                    s[kb][r] = key > lim ? -INFINITY : s[kb][r] * g.scale_log2;
                    mx = fmaxf(mx, s[kb][r]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] *= g.scale_log2;
                    mx = fmaxf(mx, s[kb][r]);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float mref = mn == -INFINITY ? 0.f : mn;
        // raw v_exp_f32: arguments are <= 0, and results below 2^-126 (flushed to zero)
        // vanish against the row maximum's 1 in both the bf16 weights and the row sum
        const float fac = __builtin_amdgcn_exp2f(m - mref);
        m = mn;
        float ls = 0.f;
        uint32_t pk[2][2][4];  // [half][k16 step][pair]
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(s[kb][8 * st + 2 * i] - mref);
                    const float p1 = __builtin_amdgcn_exp2f(s[kb][8 * st + 2 * i + 1] - mref);
                    ls += p0 + p1;
                    pk[kb][st][i] = pack_bf16x2(p0, p1);
                }
        ls += __shfl_xor(ls, 32);
        l = l * fac + ls;
        if (__ballot(fac != 1.f)) {  // some row's maximum moved: rescale its running output
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[j][e] *= fac;
        }
        // O^T += V^T P^T: P slot k of lane group hsel in step (kb, st) is key
        // 32 kb + 16 st + 8 (k / 4) + 4 hsel + k % 4 of the block
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
                        const char *pb = reinterpret_cast<const char *>(&cV[kr * VCH + ((nn >> 3) ^ ((kr & 3) << 1))]) +
                                         ((nn >> 2) & 1) * 8;
                        vf.hv[hh] =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) av4i16_t *)pb);
                    }
                    o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.v, pf, o[j], 0, 0, 0);
                }
            }
    };

    // three stages: block e landed once only block e+1's loads are younger;
    // two stages: block e+1 is issued only after the barrier, so wait for all
    auto block = [&](int e, auto Sc) __attribute__((always_inline)) {
        constexpr int S = decltype(Sc)::value;
        if constexpr (NS == 3) __builtin_amdgcn_s_waitcnt(0x0f70 | NL);  // vmcnt(NL)
        else __builtin_amdgcn_s_waitcnt(0x0f70);                          // vmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(min(e + NS - 1, npad), attn_stage<NS, S + NS - 1>(sK0, sK1, sK2),
              attn_stage<NS, S + NS - 1>(sV0, sV1, sV2));
        compute(e, attn_stage<NS, S>(sK0, sK1, sK2), attn_stage<NS, S>(sV0, sV1, sV2));
    };

    if (npad > 0) {
        issue(0, sK0, sV0);
        if constexpr (NS == 3) issue(1, sK1, sV1);
        for (int e = 0; e < npad; e += NS) {
            block(e, std::integral_constant<int, 0>{});
            block(e + 1, std::integral_constant<int, 1>{});
            if constexpr (NS == 3) block(e + 2, std::integral_constant<int, 2>{});
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load outlives the workgroup

    // lane l: query qi, columns 32 j + 8 q + 4 hsel + 0..3
    if (qi < g.Lq) {
        const float inv = 1.f / l;
        uint16_t *orow = g.O + (int64_t)h * g.o_stride + (int64_t)qi * g.ldo;
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
}

}  // namespace

hipError_t launch_attention_fwd(const AttnArgs &a, int kq, hipStream_t stream) {
    if ((kq != 64 && kq != 128) || a.H < 1 || a.Lq < 1 || a.Lk < 1 || a.group < 1 || a.H % a.group ||
        (a.causal && a.Lq > a.Lk))
        return hipErrorInvalidValue;
    const int64_t T = (int64_t)((a.Lq + 127) / 128) * a.H;
    if (T > INT32_MAX) return hipErrorInvalidValue;
    if (kq == 64)
        attn_fwd_kernel<4><<<(unsigned)T, 256, 0, stream>>>(a);
    else
        attn_fwd_kernel<8><<<(unsigned)T, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace rmm
