// C ABI of librmm: argument checks, planning, workspace layout and launch
// order for reduced matrix multiplication on gfx950 (see include/rmm.h).
//
// The path follows "Reduced Matrix Multiplication: Input-Adaptive
// Matrix-Product Reduction for LLM Inference", Sec. 3.2 and 3.3, in the
// paper's order: column norms -> TopK -> gather -> reduced product.
//
// Routes (chosen on the host from shapes and alignment, never from data):
//   MFMA    bf16, 16-byte aligned operands, leading dims and m multiples of 8:
//           colnorm_partial -> colnorm_finalize -> select -> pack A (and B^T
//           when transB) -> MFMA GEMM (-> split-K reduce when K is split).
//   DECODE  bf16, n = 1, B stored d x m, aligned: select on |a| (writes the
//           kept values) -> gathered GEMV partials -> ordered reduce.
//   GENERIC everything else (fp32, odd shapes, unaligned): the same norm and
//           select kernels, then a SIMT gathered GEMM with fp32 FMA.
// rho = 1 without RMM_FLAG_FULL_PATH keeps every index (I = [0, d)): the norm
// and select steps are skipped, idx_out receives 0..d-1, and A is used in
// place when its rows are already MFMA-ready.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "rmm_internal.h"

namespace rmm {

// ---------------------------------------------------------------- timing hooks
namespace {
struct TimingState {
    bool enabled = false;
    int capacity = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;
    std::vector<int> kind;
    int open_kind = -1;
};
TimingState g_timing;
}  // namespace

void timing_begin(hipStream_t s, int kind) {
    if (!g_timing.enabled || g_timing.used >= g_timing.capacity) {
        g_timing.open_kind = -1;
        return;
    }
    if (hipEventRecord(g_timing.ev[2 * g_timing.used], s) != hipSuccess) {
        g_timing.open_kind = -1;
        return;
    }
    g_timing.open_kind = kind;
}

void timing_end(hipStream_t s, int kind) {
    if (g_timing.open_kind != kind) return;
    if (hipEventRecord(g_timing.ev[2 * g_timing.used + 1], s) == hipSuccess) {
        g_timing.kind[g_timing.used] = kind;
        ++g_timing.used;
    }
    g_timing.open_kind = -1;
}

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t &out) {
    if (a < 0 || b < 0) return false;
    return !__builtin_mul_overflow(a, b, &out);
}

// Highest element offset touched by a strided batch of row-major matrices, +1.
bool extent(int64_t rows, int64_t cols, int64_t ld, int64_t batch, int64_t stride, int64_t &out) {
    int64_t a, c;
    if (!mul_ok(rows - 1, ld, a)) return false;
    if (!mul_ok(batch - 1, stride, c)) return false;
    if (__builtin_add_overflow(a, cols, &out)) return false;
    if (__builtin_add_overflow(out, c, &out)) return false;
    return true;
}

bool overlaps(const void *p, int64_t pbytes, const void *q, int64_t qbytes) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)pbytes;
}

enum Route { ROUTE_GENERIC = 0, ROUTE_MFMA = 1, ROUTE_DECODE = 2 };

struct Plan {
    Route route;
    int64_t k, kpad;
    bool shortcut;   // rho = 1 fast path: no norms or selection
    bool directA;    // MFMA reads A in place (no pack)
    bool transA;     // the norm pass writes A^T and the GEMM gathers its rows (no pack)
    bool fused_decode;  // decode with the selection inside the GEMV (gsplits row splits)
    ColnormPlan cp;
    GemmConfig gc;
    int gsplits;
    int64_t a_rows;  // rows of the packed A buffer per batch entry
    int64_t b_rows;  // rows of the packed B^T buffer per batch entry
    size_t off_part, off_s, off_idx, off_Ap, off_At, off_Bp, off_gpart, off_aval, total;
};

// Largest output width for which the A^T route is taken.  It replaces the
// pack pass by a second write of A in the norm pass, and its two-operand
// GEMM runs a K step as fast as the operand-block kernels up to m = 4096 and
// 0.7% slower at m = 28672 (MI355X): on a 4096 x 8192 block the pack costs
// 28 us and the extra write 15 us, so the route still gains ~5 us on a
// 4096 x 8192 x 28672 product and would break even near m = 57000.
constexpr int64_t kTransAMaxM = 32768;

// Host-side rho -> k (Sec. 3.2); see rmm_k in rmm.h for the rounding rule.
int64_t k_of(double rho, int64_t d) {
    if (!(rho > 0.0) || !(rho <= 1.0) || d < 1) return 0;
    const double p = rho * (double)d;
    const double r = nearbyint(p);
    const double tol = 1e-9 * (p > 1.0 ? p : 1.0);
    double kk = fabs(p - r) <= tol ? r : ceil(p);
    if (kk < 1.0) kk = 1.0;
    if (kk > (double)d) kk = (double)d;
    return (int64_t)kk;
}

// Validates the descriptor; fills element extents of A, B, Y.
rmm_status_t check_desc(const rmm_desc_t *ds, int64_t &extA, int64_t &extB, int64_t &extY) {
    if (!ds) return RMM_ERR_INVALID_ARG;
    if (ds->dtype != RMM_F32 && ds->dtype != RMM_BF16) return RMM_ERR_INVALID_ARG;
    if (ds->transB != 0 && ds->transB != 1) return RMM_ERR_INVALID_ARG;
    if (ds->n < 1 || ds->d < 1 || ds->m < 1 || ds->batch < 1 || ds->b_group < 1) return RMM_ERR_INVALID_ARG;
    if (ds->d > INT32_MAX) return RMM_ERR_INVALID_ARG;
    if (ds->batch > 65535 || ds->n > INT32_MAX / 2 || ds->m > INT32_MAX / 2) return RMM_ERR_INVALID_ARG;
    if (ds->lda < ds->d || ds->ldy < ds->m) return RMM_ERR_INVALID_ARG;
    if (ds->ldb < (ds->transB ? ds->d : ds->m)) return RMM_ERR_INVALID_ARG;
    if (ds->strideA < 0 || ds->strideB < 0 || ds->strideY < 0) return RMM_ERR_INVALID_ARG;
    if (!isfinite(ds->alpha)) return RMM_ERR_INVALID_ARG;
    if ((ds->flags & ~RMM_FLAG_FULL_PATH) != 0) return RMM_ERR_INVALID_ARG;
    const int64_t nb = (ds->batch + ds->b_group - 1) / ds->b_group;
    if (!extent(ds->n, ds->d, ds->lda, ds->batch, ds->strideA, extA)) return RMM_ERR_INVALID_ARG;
    if (!extent(ds->transB ? ds->m : ds->d, ds->transB ? ds->d : ds->m, ds->ldb, nb, ds->strideB, extB))
        return RMM_ERR_INVALID_ARG;
    if (!extent(ds->n, ds->m, ds->ldy, ds->batch, ds->strideY, extY)) return RMM_ERR_INVALID_ARG;
    // batch entries must not write overlapping outputs
    if (ds->batch > 1) {
        int64_t one;
        if (!extent(ds->n, ds->m, ds->ldy, 1, 0, one)) return RMM_ERR_INVALID_ARG;
        if (ds->strideY < one) return RMM_ERR_INVALID_ARG;
    }
    return RMM_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The MFMA route addresses each operand with 32-bit byte offsets from a
// per-entry base (buffer loads); every operand extent must stay below 2^31.
constexpr int64_t kMaxBufferBytes = 0x7fffffffLL;
int64_t a_extent_bytes(const rmm_desc_t *ds) { return ((ds->n - 1) * ds->lda + ds->d) * 2; }
int64_t b_extent_bytes(const rmm_desc_t *ds) {
    return ds->transB ? ((ds->m - 1) * ds->ldb + ds->d) * 2 : ((ds->d - 1) * ds->ldb + ds->m) * 2;
}
bool mfma_extents_ok(const rmm_desc_t *ds, int64_t kpad) {
    return a_extent_bytes(ds) < kMaxBufferBytes && b_extent_bytes(ds) < kMaxBufferBytes &&
           (ds->n + 31) / 32 * 32 * kpad * 2 < kMaxBufferBytes && ds->m * kpad * 2 < kMaxBufferBytes;
}

// Alignment-based part of the route choice; pointers may be null when only
// sizing (then alignment is assumed, which can only over-size).
Plan make_plan(const rmm_desc_t *ds, int64_t k, const void *A, const void *B, const void *Y, bool given = false) {
    Plan p;
    memset(&p, 0, sizeof(p));
    p.k = k;
    // The MFMA kernel runs an even number of 64-wide K steps; the padded
    // columns of packed operands are zero and padded index entries are -1.
    p.kpad = (k + 127) / 128 * 128;
    p.shortcut = !given && (k == ds->d) && !(ds->flags & RMM_FLAG_FULL_PATH);
    const bool bf = ds->dtype == RMM_BF16;
    const bool ptr_ok = (!A || aligned16(A)) && (!B || aligned16(B)) && (!Y || aligned16(Y));
    const bool ld_ok = ds->lda % 8 == 0 && ds->ldb % 8 == 0 && ds->ldy % 8 == 0 && ds->m % 8 == 0 &&
                       (ds->batch == 1 || (ds->strideA % 8 == 0 && ds->strideB % 8 == 0 && ds->strideY % 8 == 0));
    if (bf && ptr_ok && ld_ok && ds->n == 1 && !ds->transB && ds->batch == 1 && ds->d <= kFusedSelectMaxD) {
        p.route = ROUTE_DECODE;
        p.shortcut = false;  // the fused |a| selection also produces the kept values
        // wide outputs: every GEMV workgroup selects from |a| itself (no select launch)
        p.fused_decode = !given && ds->m >= decode_fused_min_m();
        if (p.fused_decode) {
            p.gsplits = decode_fused_splits(0, ds->m, k);
            p.off_gpart = 0;
            p.total = p.gsplits > 1 ? align_up((size_t)p.gsplits * ds->m * 4) : 0;
            return p;
        }
    } else if (bf && ptr_ok && ld_ok && mfma_extents_ok(ds, p.kpad)) {
        p.route = ROUTE_MFMA;
    } else {
        p.route = ROUTE_GENERIC;
    }

    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align_up(bytes);
        return o;
    };
    const int64_t batch = ds->batch, d = ds->d, n = ds->n, m = ds->m;
    const bool norms = !given && !p.shortcut && p.route != ROUTE_DECODE;
    // narrow output (attention's P V: m = d_v): A read in place, its kept
    // columns gathered inside the GEMM, so no pack of A[:, I]
    const bool gcol = p.route == ROUTE_MFMA && !ds->transB && m <= kGcolMaxM && n >= 128 && d <= kGcolMaxD &&
                      d % 8 == 0 && a_extent_bytes(ds) < kMaxBufferBytes;
    // A^T route: one bf16 product of at most kTransAMaxM output columns with
    // B stored d x m, whose norms are computed anyway
    if (!gcol && p.route == ROUTE_MFMA && norms && batch == 1 && !ds->transB && m <= kTransAMaxM && n % 8 == 0 &&
        d % 8 == 0 && n * d * 2 < kMaxBufferBytes) {
        p.gc = gemm_choose_transposed(n, m, k, d);
        p.transA = p.gc.tile == 5;
    }
    if (norms) {
        p.cp = p.transA ? colnorm_transpose_plan(n, d) : colnorm_plan(ds->dtype, n, d, batch);
        p.off_part = take((size_t)p.cp.chunks * d * batch * 4);
        p.off_s = take((size_t)d * batch * 4);
    }
    // the streaming kernel runs one or two whole 64-entry K steps
    if (p.route == ROUTE_MFMA && gemm_choose(n, m, k, batch, d, ds->transB).tile == 3) p.kpad = k <= 64 ? 64 : 128;
    p.off_idx = take((size_t)p.kpad * batch * 4);  // padded index rows (-1 beyond k)
    if (gcol) {
        p.gc.tile = 6;
        p.gc.splits = 1;
    } else if (p.transA) {
        p.off_At = take((size_t)d * n * 2);
        if (p.gc.splits > 1) p.off_gpart = take((size_t)p.gc.splits * n * m * 4);
    } else if (p.route == ROUTE_MFMA) {
        p.gc = gemm_choose(n, m, k, batch, d, ds->transB);
        const bool blocks = p.gc.tile >= 2;  // operands in MFMA operand blocks
        if (p.gc.tile == 3) p.kpad = k <= 64 ? 64 : 128;
        p.directA = p.shortcut && d % 128 == 0 && !blocks;
        p.a_rows = blocks ? (n + 31) / 32 * 32 : n;  // operand blocks cover whole 32-row groups
        p.b_rows = p.gc.tile == 3 ? (m + 31) / 32 * 32 : m;
        if (!p.directA) p.off_Ap = take((size_t)batch * p.a_rows * p.kpad * 2);
        if (ds->transB) p.off_Bp = take((size_t)batch * p.b_rows * p.kpad * 2);
        if (p.gc.splits > 1) p.off_gpart = take((size_t)p.gc.splits * batch * n * m * 4);
    } else if (p.route == ROUTE_DECODE) {
        p.gsplits = gemv_splits(m, k);
        p.off_aval = take((size_t)k * 4);
        p.off_gpart = take((size_t)p.gsplits * m * 4);
    }
    p.total = off;
    return p;
}

thread_local hipError_t g_last_error = hipSuccess;

rmm_status_t run_matmul(const rmm_desc_t *desc, const void *A, const void *B, int64_t k, const int32_t *idx_in,
                        void *Y, int32_t *idx_out, void *workspace, size_t ws_bytes, hipStream_t stream,
                        int64_t extA, int64_t extB, int64_t extY);

// ------------------------------------------------------------------ gated MLP block
struct MlpPlan {
    int64_t k_in, kpad_in, k_h, kpad_h, chunks_h;
    ColnormPlan cp;
    GemmConfig gc, gc_h;
    size_t off_part, off_idx, off_xt, off_ht, off_hpart, off_idx_h, off_gpart, total;
};

rmm_status_t mlp_plan(const void *x, const void *Wgu, const void *Wd, int64_t n, int64_t d, int64_t m, double rho_in,
                      double rho_h, MlpPlan &p) {
    memset(&p, 0, sizeof(p));
    if (n < 1 || d < 1 || m < 1) return RMM_ERR_INVALID_ARG;
    p.k_in = k_of(rho_in, d);
    p.k_h = k_of(rho_h, m);
    if (p.k_in < 1 || p.k_h < 1) return RMM_ERR_INVALID_ARG;
    if (n % 8 || d % 8 || m % 32 || 2 * m > kTransAMaxM || n * d * 2 >= kMaxBufferBytes ||
        d * 2 * m * 2 >= kMaxBufferBytes || n * m * 2 >= kMaxBufferBytes || m * d * 2 >= kMaxBufferBytes ||
        (x && !aligned16(x)) || (Wgu && !aligned16(Wgu)) || (Wd && !aligned16(Wd)))
        return RMM_ERR_UNSUPPORTED;
    p.kpad_in = (p.k_in + 127) / 128 * 128;
    // the two-operand kernel at any size, over one K range (SwiGLU needs whole sums)
    if (!gemm_tdma_fits(p.kpad_in, 1, d)) return RMM_ERR_UNSUPPORTED;
    p.gc.tile = 5;
    p.gc.splits = 1;
    p.cp = colnorm_transpose_plan(n, d);
    // Down: h^T and the column sums of h^2 per 256-row chunk come from the
    // SwiGLU epilogue; its selection, then the two-operand GEMM over h^T rows
    p.kpad_h = (p.k_h + 127) / 128 * 128;
    p.chunks_h = (n + 255) / 256;
    p.gc_h = gemm_choose_transposed(n, d, p.k_h, m);
    if (p.gc_h.tile != 5) {
        // few output tiles (a short block of tokens): the two-operand kernel
        // with as many K splits as fill the chip (at least 16 K steps each)
        // and at least as many as its LDS row list needs
        const int64_t tiles = ((n + 255) / 256) * ((d + 255) / 256), ksteps = p.kpad_h / 64;
        int64_t s = std::min((256 + tiles - 1) / tiles, ksteps / 16);
        if (s < 1) s = 1;
        while (s < 64 && !gemm_tdma_fits(p.kpad_h, (int)s, m)) ++s;
        if (!gemm_tdma_fits(p.kpad_h, (int)s, m)) return RMM_ERR_UNSUPPORTED;
        p.gc_h.tile = 5;
        p.gc_h.splits = (int)s;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align_up(bytes);
        return o;
    };
    p.off_part = take((size_t)p.cp.chunks * d * 4 + (size_t)d * 4);  // partials, then s
    p.off_idx = take((size_t)p.kpad_in * 4);
    p.off_xt = take((size_t)d * n * 2);
    p.off_ht = take((size_t)m * n * 2);
    p.off_hpart = take((size_t)p.chunks_h * m * 4 + (size_t)m * 4);  // partials, then s of h
    p.off_idx_h = take((size_t)p.kpad_h * 4);
    if (p.gc_h.splits > 1) p.off_gpart = take((size_t)p.gc_h.splits * n * d * 4);
    p.total = off;
    return RMM_OK;
}


#define RMM_LAUNCH(kind, call)              \
    do {                                    \
        timing_begin(stream, kind);         \
        hipError_t e_ = (call);             \
        timing_end(stream, kind);           \
        if (e_ != hipSuccess) {             \
            g_last_error = e_;              \
            return RMM_ERR_HIP;             \
        }                                   \
    } while (0)

}  // namespace
}  // namespace rmm

using namespace rmm;

extern "C" {

int64_t rmm_k(double rho, int64_t d) { return k_of(rho, d); }

int32_t rmm_version(void) { return 100; }

const char *rmm_last_hip_error(void) { return hipGetErrorString(g_last_error); }

const char *rmm_status_string(rmm_status_t s) {
    switch (s) {
        case RMM_OK: return "ok";
        case RMM_ERR_INVALID_ARG: return "invalid argument";
        case RMM_ERR_UNSUPPORTED: return "unsupported";
        case RMM_ERR_WORKSPACE: return "workspace missing or too small";
        case RMM_ERR_HIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

void rmm_desc_init(rmm_desc_t *ds, rmm_dtype_t dtype, int64_t n, int64_t d, int64_t m) {
    if (!ds) return;
    memset(ds, 0, sizeof(*ds));
    ds->dtype = dtype;
    ds->n = n;
    ds->d = d;
    ds->m = m;
    ds->lda = d;
    ds->ldb = m;
    ds->ldy = m;
    ds->batch = 1;
    ds->b_group = 1;
    ds->alpha = 1.0f;
}

size_t rmm_colnorm_workspace_size(rmm_dtype_t dt, int64_t n, int64_t d) {
    if ((dt != RMM_F32 && dt != RMM_BF16) || n < 1 || d < 1) return SIZE_MAX;
    ColnormPlan p = colnorm_plan(dt, n, d, 1);
    return (size_t)p.chunks * (size_t)d * 4;
}

rmm_status_t rmm_colnorm(const void *A, rmm_dtype_t dt, int64_t n, int64_t d, int64_t lda, float *s_out,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!A || !s_out || (dt != RMM_F32 && dt != RMM_BF16) || n < 1 || d < 1 || lda < d) return RMM_ERR_INVALID_ARG;
    int64_t ext;
    if (!extent(n, d, lda, 1, 0, ext) || n > INT32_MAX / 2) return RMM_ERR_INVALID_ARG;
    ColnormPlan p = colnorm_plan(dt, n, d, 1);
    const size_t need = (size_t)p.chunks * (size_t)d * 4;
    if (ws_bytes < need || !workspace) return RMM_ERR_WORKSPACE;
    float *part = static_cast<float *>(workspace);
    RMM_LAUNCH(RMM_KERNEL_COLNORM, launch_colnorm_partial(A, dt, n, d, lda, 1, 0, p, part, stream));
    RMM_LAUNCH(RMM_KERNEL_FINALIZE,
               launch_colnorm_finalize(part, p.chunks, d, 1, s_out, stream));
    return RMM_OK;
}

rmm_status_t rmm_select(const float *s, int64_t batch, int64_t d, int64_t k, int32_t *idx_out, hipStream_t stream) {
    if (!s || !idx_out || batch < 1 || batch > 65535 || d < 1 || d > INT32_MAX || k < 1 || k > d)
        return RMM_ERR_INVALID_ARG;
    RMM_LAUNCH(RMM_KERNEL_SELECT,
               launch_select(s, nullptr, RMM_F32, 0, batch, d, k, idx_out, k, nullptr, 0, nullptr, stream));
    return RMM_OK;
}

size_t rmm_workspace_size(const rmm_desc_t *desc, double rho) {
    int64_t ea, eb, ey;
    if (check_desc(desc, ea, eb, ey) != RMM_OK) return SIZE_MAX;
    const int64_t k = k_of(rho, desc->d);
    if (k < 1) return SIZE_MAX;
    return make_plan(desc, k, nullptr, nullptr, nullptr).total;
}

rmm_status_t rmm_plan_info(const rmm_desc_t *desc, double rho, int32_t *info) {
    int64_t ea, eb, ey;
    if (!info || check_desc(desc, ea, eb, ey) != RMM_OK) return RMM_ERR_INVALID_ARG;
    const int64_t k = k_of(rho, desc->d);
    if (k < 1) return RMM_ERR_INVALID_ARG;
    const Plan p = make_plan(desc, k, nullptr, nullptr, nullptr);
    info[0] = p.route;
    info[1] = p.route == ROUTE_MFMA ? p.gc.tile : -1;
    info[2] = p.route == ROUTE_MFMA ? p.gc.splits : p.route == ROUTE_DECODE ? p.gsplits : 1;
    return RMM_OK;
}

rmm_status_t rmm_matmul(const rmm_desc_t *desc, const void *A, const void *B, double rho, void *Y,
                        int32_t *idx_out, void *workspace, size_t ws_bytes, hipStream_t stream) {
    int64_t extA, extB, extY;
    rmm_status_t st = check_desc(desc, extA, extB, extY);
    if (st != RMM_OK) return st;
    if (!A || !B || !Y) return RMM_ERR_INVALID_ARG;
    const int64_t k = k_of(rho, desc->d);
    if (k < 1) return RMM_ERR_INVALID_ARG;
    return run_matmul(desc, A, B, k, nullptr, Y, idx_out, workspace, ws_bytes, stream, extA, extB, extY);
}

size_t rmm_workspace_size_indexed(const rmm_desc_t *desc, int64_t k) {
    int64_t ea, eb, ey;
    if (check_desc(desc, ea, eb, ey) != RMM_OK || k < 1 || k > desc->d) return SIZE_MAX;
    return make_plan(desc, k, nullptr, nullptr, nullptr, true).total;
}

rmm_status_t rmm_matmul_indexed(const rmm_desc_t *desc, const void *A, const void *B, const int32_t *idx,
                                int64_t k, void *Y, void *workspace, size_t ws_bytes, hipStream_t stream) {
    int64_t extA, extB, extY;
    rmm_status_t st = check_desc(desc, extA, extB, extY);
    if (st != RMM_OK) return st;
    if (!A || !B || !Y || !idx || k < 1 || k > desc->d) return RMM_ERR_INVALID_ARG;
    return run_matmul(desc, A, B, k, idx, Y, nullptr, workspace, ws_bytes, stream, extA, extB, extY);
}

rmm_status_t rmm_gated_weights(const void *Wg, const void *Wu, int64_t d, int64_t m, int32_t transposed, void *Wgu,
                               hipStream_t stream) {
    if (!Wg || !Wu || !Wgu || d < 1 || m < 32 || m % 32 || (transposed != 0 && transposed != 1) ||
        !aligned16(Wgu) || d * 2 * m * 2 >= kMaxBufferBytes)
        return RMM_ERR_INVALID_ARG;
    RMM_LAUNCH(RMM_KERNEL_OTHER, launch_gated_weights(static_cast<const uint16_t *>(Wg),
                                                      static_cast<const uint16_t *>(Wu), d, m, transposed,
                                                      static_cast<uint16_t *>(Wgu), stream));
    return RMM_OK;
}

size_t rmm_gated_mlp_workspace_size(int64_t n, int64_t d, int64_t m, double rho_in, double rho_h) {
    MlpPlan p;
    if (mlp_plan(nullptr, nullptr, nullptr, n, d, m, rho_in, rho_h, p) != RMM_OK) return SIZE_MAX;
    return p.total;
}

rmm_status_t rmm_gated_mlp(const void *x, const void *Wgu, const void *Wd, int64_t n, int64_t d, int64_t m,
                           double rho_in, double rho_h, void *Y, void *h_out, int32_t *idx_in_out,
                           int32_t *idx_h_out, void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!x || !Wgu || !Wd || !Y) return RMM_ERR_INVALID_ARG;
    MlpPlan p;
    rmm_status_t st = mlp_plan(x, Wgu, Wd, n, d, m, rho_in, rho_h, p);
    if (st != RMM_OK) return st;
    if (!aligned16(Y) || (h_out && !aligned16(h_out))) return RMM_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < p.total) return RMM_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255) return RMM_ERR_INVALID_ARG;
    char *ws = static_cast<char *>(workspace);
    const int64_t xb = n * d * 2, wb = d * 2 * m * 2, db = m * d * 2, yb = n * d * 2, hb = n * m * 2;
    if (overlaps(Y, yb, x, xb) || overlaps(Y, yb, Wgu, wb) || overlaps(Y, yb, Wd, db) ||
        overlaps(ws, (int64_t)p.total, x, xb) || overlaps(ws, (int64_t)p.total, Wgu, wb) ||
        overlaps(ws, (int64_t)p.total, Wd, db) || overlaps(ws, (int64_t)p.total, Y, yb) ||
        (h_out && (overlaps(h_out, hb, x, xb) || overlaps(h_out, hb, Y, yb) || overlaps(h_out, hb, ws, (int64_t)p.total) ||
                   overlaps(h_out, hb, Wgu, wb) || overlaps(h_out, hb, Wd, db))) ||
        (idx_in_out && (overlaps(idx_in_out, p.k_in * 4, Y, yb) || overlaps(idx_in_out, p.k_in * 4, ws, (int64_t)p.total))) ||
        (idx_h_out && (overlaps(idx_h_out, p.k_h * 4, Y, yb) || overlaps(idx_h_out, p.k_h * 4, ws, (int64_t)p.total))))
        return RMM_ERR_INVALID_ARG;
    float *part = reinterpret_cast<float *>(ws + p.off_part);
    int32_t *pidx = reinterpret_cast<int32_t *>(ws + p.off_idx);
    uint16_t *xt = reinterpret_cast<uint16_t *>(ws + p.off_xt);
    uint16_t *ht = reinterpret_cast<uint16_t *>(ws + p.off_ht);
    float *hpart = reinterpret_cast<float *>(ws + p.off_hpart);
    int32_t *pidx_h = reinterpret_cast<int32_t *>(ws + p.off_idx_h);
    // Up and Gate: one norm pass (also writing x^T), one selection (the same input gives the same set)
    RMM_LAUNCH(RMM_KERNEL_COLNORM, launch_colnorm_transpose(x, n, d, d, p.cp, xt, n, part, stream));
    if (norm_select_ok(p.cp.chunks, d)) {
        RMM_LAUNCH(RMM_KERNEL_SELECT,
                   launch_norm_select(part, p.cp.chunks, d, 1, p.k_in, idx_in_out, p.k_in, pidx, p.kpad_in, stream));
    } else {
        float *s = part + p.cp.chunks * d;
        RMM_LAUNCH(RMM_KERNEL_FINALIZE, launch_colnorm_finalize(part, p.cp.chunks, d, 1, s, stream));
        RMM_LAUNCH(RMM_KERNEL_SELECT, launch_select(s, nullptr, RMM_F32, 0, 1, d, p.k_in, idx_in_out, p.k_in, pidx,
                                                    p.kpad_in, nullptr, stream));
    }
    // h = SiLU(x_I Wg_I) * (x_I Wu_I): one GEMM over the interleaved operand, SwiGLU in its epilogue,
    // which writes h^T and the column sums of h^2 (and h itself when asked for)
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A = xt;
    g.lda = n;
    g.a_bytes = d * n * 2;
    g.B = static_cast<const uint16_t *>(Wgu);
    g.ldb = 2 * m;
    g.b_bytes = wb;
    g.group = 1;
    g.bmode = 0;
    g.idx = pidx;
    g.ld_idx = p.kpad_in;
    g.Y = static_cast<uint16_t *>(h_out);
    g.ldy = m;
    g.Yt = ht;
    g.npart = hpart;
    g.n = n;
    g.m = 2 * m;
    g.k = p.k_in;
    g.kpad = p.kpad_in;
    g.batch = 1;
    g.alpha = 1.f;
    g.splits = 1;
    g.epi = 1;
    RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_bf16(g, p.gc, stream));
    // Down: h's column norms from the epilogue's partials, its own selection, rows of h^T and Wd
    if (norm_select_ok(p.chunks_h, m)) {
        RMM_LAUNCH(RMM_KERNEL_SELECT,
                   launch_norm_select(hpart, p.chunks_h, m, 1, p.k_h, idx_h_out, p.k_h, pidx_h, p.kpad_h, stream));
    } else {
        float *sh = hpart + p.chunks_h * m;
        RMM_LAUNCH(RMM_KERNEL_FINALIZE, launch_colnorm_finalize(hpart, p.chunks_h, m, 1, sh, stream));
        RMM_LAUNCH(RMM_KERNEL_SELECT, launch_select(sh, nullptr, RMM_F32, 0, 1, m, p.k_h, idx_h_out, p.k_h, pidx_h,
                                                    p.kpad_h, nullptr, stream));
    }
    GemmArgs gd;
    memset(&gd, 0, sizeof(gd));
    gd.A = ht;
    gd.lda = n;
    gd.a_bytes = m * n * 2;
    gd.B = static_cast<const uint16_t *>(Wd);
    gd.ldb = d;
    gd.b_bytes = db;
    gd.group = 1;
    gd.bmode = 0;
    gd.idx = pidx_h;
    gd.ld_idx = p.kpad_h;
    gd.Y = static_cast<uint16_t *>(Y);
    gd.ldy = d;
    gd.n = n;
    gd.m = d;
    gd.k = p.k_h;
    gd.kpad = p.kpad_h;
    gd.batch = 1;
    gd.alpha = 1.f;
    gd.splits = p.gc_h.splits;
    gd.part = p.gc_h.splits > 1 ? reinterpret_cast<float *>(ws + p.off_gpart) : nullptr;
    RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_bf16(gd, p.gc_h, stream));
    if (p.gc_h.splits > 1)
        RMM_LAUNCH(RMM_KERNEL_REDUCE, launch_splitk_reduce(gd.part, p.gc_h.splits, n, d, 1, 1.f,
                                                           static_cast<uint16_t *>(Y), d, 0, stream));
    return RMM_OK;
}

namespace {
struct AttnPlan {
    int64_t k, kpad, qrows, krows;
    ColnormPlan cp;
    size_t off_part, off_s, off_idx, off_k, total;
};

rmm_status_t attn_plan(int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t dh, double rho, AttnPlan &p) {
    memset(&p, 0, sizeof(p));
    if (H < 1 || Hkv < 1 || Lq < 1 || Lk < 1 || dh < 1 || H % Hkv) return RMM_ERR_INVALID_ARG;
    p.k = k_of(rho, dh);
    if (p.k < 1) return RMM_ERR_INVALID_ARG;
    if (dh > 128 || dh % 8 || H > 65535) return RMM_ERR_UNSUPPORTED;
    p.kpad = p.k <= 64 ? 64 : 128;
    p.qrows = (Lq + 31) / 32 * 32;
    p.krows = (Lk + 31) / 32 * 32;
    if (p.qrows * p.kpad * 2 >= kMaxBufferBytes || p.krows * p.kpad * 2 >= kMaxBufferBytes ||
        Lk * 128 * 2 >= kMaxBufferBytes || Lq * dh * 2 >= kMaxBufferBytes || Lk * dh * 2 >= kMaxBufferBytes)
        return RMM_ERR_UNSUPPORTED;
    p.cp = colnorm_plan(RMM_BF16, Lq, dh, H);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align_up(bytes);
        return o;
    };
    p.off_part = take((size_t)p.cp.chunks * dh * H * 4);
    p.off_s = take((size_t)dh * H * 4);
    p.off_idx = take((size_t)p.kpad * H * 4);
    p.off_k = take((size_t)H * p.krows * p.kpad * 2);
    p.total = off;
    return RMM_OK;
}
}  // namespace

size_t rmm_attention_workspace_size(int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t dh, double rho) {
    AttnPlan p;
    return attn_plan(H, Hkv, Lq, Lk, dh, rho, p) == RMM_OK ? p.total : SIZE_MAX;
}

rmm_status_t rmm_attention(const void *q, const void *k, const void *v, int64_t H, int64_t Hkv, int64_t Lq,
                           int64_t Lk, int64_t dh, int64_t dv, double rho, int32_t causal, void *out, int32_t *idx_out,
                           void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !out || (causal != 0 && causal != 1)) return RMM_ERR_INVALID_ARG;
    AttnPlan p;
    rmm_status_t st = attn_plan(H, Hkv, Lq, Lk, dh, rho, p);
    if (st != RMM_OK) return st;
    if (causal && Lq > Lk) return RMM_ERR_INVALID_ARG;
    if (dv != 128 || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RMM_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < p.total) return RMM_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255) return RMM_ERR_INVALID_ARG;
    const int64_t qb = H * Lq * dh * 2, kb = Hkv * Lk * dh * 2, vb = Hkv * Lk * dv * 2, ob = H * Lq * dv * 2;
    char *ws = static_cast<char *>(workspace);
    const int64_t wb = (int64_t)p.total;
    if (overlaps(out, ob, q, qb) || overlaps(out, ob, k, kb) || overlaps(out, ob, v, vb) || overlaps(ws, wb, q, qb) ||
        overlaps(ws, wb, k, kb) || overlaps(ws, wb, v, vb) || overlaps(ws, wb, out, ob) ||
        (idx_out && (overlaps(idx_out, H * p.k * 4, out, ob) || overlaps(idx_out, H * p.k * 4, ws, wb) ||
                     overlaps(idx_out, H * p.k * 4, q, qb) || overlaps(idx_out, H * p.k * 4, k, kb) ||
                     overlaps(idx_out, H * p.k * 4, v, vb))))
        return RMM_ERR_INVALID_ARG;
    float *part = reinterpret_cast<float *>(ws + p.off_part);
    float *s = reinterpret_cast<float *>(ws + p.off_s);
    int32_t *pidx = reinterpret_cast<int32_t *>(ws + p.off_idx);
    uint16_t *Kp = reinterpret_cast<uint16_t *>(ws + p.off_k);
    // the dimensions each query head keeps: TopK of its columns' norms (one per head)
    RMM_LAUNCH(RMM_KERNEL_COLNORM, launch_colnorm_partial(q, RMM_BF16, Lq, dh, dh, H, Lq * dh, p.cp, part, stream));
    // per query head K_g[:, I_h] in MFMA operand blocks (Q's kept columns are gathered in the kernel)
    if (select_pack_short_ok(dh, p.k, p.kpad, p.cp.chunks)) {
        // every pack workgroup ranks its head's norms itself: no selection launch
        RMM_LAUNCH(RMM_KERNEL_PACK, launch_select_pack_short(part, p.cp.chunks, p.k, idx_out, p.k, pidx, p.kpad, k, Lk,
                                                             dh, dh, Lk * dh, H / Hkv, Kp, p.krows * p.kpad, H,
                                                             stream));
    } else {
        if (norm_select_ok(p.cp.chunks, dh)) {
            RMM_LAUNCH(RMM_KERNEL_SELECT,
                       launch_norm_select(part, p.cp.chunks, dh, H, p.k, idx_out, p.k, pidx, p.kpad, stream));
        } else {
            RMM_LAUNCH(RMM_KERNEL_FINALIZE, launch_colnorm_finalize(part, p.cp.chunks, dh, H, s, stream));
            RMM_LAUNCH(RMM_KERNEL_SELECT,
                       launch_select(s, nullptr, RMM_F32, 0, H, dh, p.k, idx_out, p.k, pidx, p.kpad, nullptr, stream));
        }
        RMM_LAUNCH(RMM_KERNEL_PACK, launch_pack(k, RMM_BF16, Lk, dh, dh, Lk * dh, H / Hkv, pidx, p.kpad, p.kpad, Kp,
                                                p.krows * p.kpad, H, 1, stream));
    }
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.Q = static_cast<const uint16_t *>(q);
    a.idx = pidx;
    a.ld_idx = p.kpad;
    a.dh = dh;
    a.K = Kp;
    a.k_stride = p.krows * p.kpad;
    a.k_bytes = p.krows * p.kpad * 2;
    a.V = static_cast<const uint16_t *>(v);
    a.ldv = dv;
    a.v_stride = Lk * dv;
    a.v_bytes = Lk * dv * 2;
    a.O = static_cast<uint16_t *>(out);
    a.ldo = dv;
    a.o_stride = Lq * dv;
    a.H = (int)H;
    a.group = (int)(H / Hkv);
    a.Lq = (int)Lq;
    a.Lk = (int)Lk;
    a.causal = causal;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)dh));
    RMM_LAUNCH(RMM_KERNEL_GEMM, launch_attention_fwd(a, (int)p.kpad, stream));
    return RMM_OK;
}

size_t rmm_decode_wq_workspace_size(int64_t d, int64_t m, double rho) {
    const int64_t k = k_of(rho, d);
    if (k < 1 || d > kFusedSelectMaxD || m < 16 || m % 16) return SIZE_MAX;
    if (m >= decode_fused_min_m()) {  // the selection inside the GEMV: only the split partials
        const int s = decode_fused_splits(1, m, k);
        return s > 1 ? align_up((size_t)s * m * 4) : 0;
    }
    const int64_t kpad = (k + 127) / 128 * 128;
    const int splits = gemv_wq_splits(m, k);
    return align_up((size_t)kpad * 4) + align_up((size_t)k * 4) + align_up((size_t)splits * m * 4);
}

rmm_status_t rmm_decode_wq(const void *a, const void *Bq, int32_t fmt, const float *scale, int64_t d, int64_t m,
                           int64_t ldb, double rho, float alpha, void *y, int32_t *idx_out, void *workspace,
                           size_t ws_bytes, hipStream_t stream) {
    if (!a || !Bq || !scale || !y || (fmt != RMM_WQ_FP8_E4M3 && fmt != RMM_WQ_INT8)) return RMM_ERR_INVALID_ARG;
    const int64_t k = k_of(rho, d);
    if (k < 1 || d < 1 || m < 1 || ldb < m) return RMM_ERR_INVALID_ARG;
    if (d > kFusedSelectMaxD || m % 16 || ldb % 16 || !aligned16(a) || !aligned16(Bq) || !aligned16(y) ||
        ((uintptr_t)scale & 3))
        return RMM_ERR_UNSUPPORTED;
    const size_t need = rmm_decode_wq_workspace_size(d, m, rho);
    if (need > 0 && (!workspace || ws_bytes < need)) return RMM_ERR_WORKSPACE;
    if (need > 0 && ((uintptr_t)workspace & 255)) return RMM_ERR_INVALID_ARG;
    const int64_t ab = d * 2, bb = (d - 1) * ldb + m, sb = m * 4, yb = m * 2;
    char *ws = static_cast<char *>(workspace);
    if (overlaps(y, yb, a, ab) || overlaps(y, yb, Bq, bb) || overlaps(y, yb, scale, sb) ||
        overlaps(ws, (int64_t)need, a, ab) || overlaps(ws, (int64_t)need, Bq, bb) ||
        overlaps(ws, (int64_t)need, scale, sb) || overlaps(ws, (int64_t)need, y, yb) ||
        (idx_out && (overlaps(idx_out, k * 4, y, yb) || overlaps(idx_out, k * 4, ws, (int64_t)need) ||
                     overlaps(idx_out, k * 4, a, ab) || overlaps(idx_out, k * 4, Bq, bb))))
        return RMM_ERR_INVALID_ARG;
    if (m >= decode_fused_min_m()) {
        // the |a| selection inside every GEMV workgroup, then the split sum (if split)
        const int fs = decode_fused_splits(1, m, k);
        float *fpart = reinterpret_cast<float *>(ws);
        RMM_LAUNCH(RMM_KERNEL_GEMV, launch_decode_fused(static_cast<const uint16_t *>(a), d, k, Bq,
                                                        fmt == RMM_WQ_FP8_E4M3 ? 1 : 2, ldb, m, scale, alpha,
                                                        static_cast<uint16_t *>(y), idx_out, fs, fpart, stream));
        if (fs > 1)
            RMM_LAUNCH(RMM_KERNEL_REDUCE,
                       launch_splitk_reduce(fpart, fs, 1, m, 1, alpha, static_cast<uint16_t *>(y), m, 0, stream));
        return RMM_OK;
    }
    const int64_t kpad = (k + 127) / 128 * 128;
    const int splits = gemv_wq_splits(m, k);
    int32_t *pidx = reinterpret_cast<int32_t *>(ws);
    float *aval = reinterpret_cast<float *>(ws + align_up((size_t)kpad * 4));
    float *gpart = reinterpret_cast<float *>(ws + align_up((size_t)kpad * 4) + align_up((size_t)k * 4));
    // the kept rows I = TopK(|a_j|) with their values, the 8-bit GEMV, the split sum
    RMM_LAUNCH(RMM_KERNEL_SELECT, launch_select(nullptr, a, RMM_BF16, 0, 1, d, k, idx_out, k, pidx, kpad, aval, stream));
    RMM_LAUNCH(RMM_KERNEL_GEMV, launch_gemv_wq_partial(static_cast<const uint8_t *>(Bq), fmt, ldb, m, scale, pidx,
                                                       aval, k, splits, gpart, stream));
    RMM_LAUNCH(RMM_KERNEL_REDUCE,
               launch_splitk_reduce(gpart, splits, 1, m, 1, alpha, static_cast<uint16_t *>(y), m, 0, stream));
    return RMM_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- reduced product over 8-bit weights
namespace rmm {
namespace {
struct WqPlan {
    int64_t k, kpad;
    ColnormPlan cp;
    GemmConfig gc;
    size_t off_part, off_s, off_idx, off_At, off_gpart, total;
};

// n > 1: the transposing norm pass, the selection, then the two-operand GEMM
// over rows of A^T and 8-bit rows of B (one K range per split).
rmm_status_t wq_plan(int64_t n, int64_t d, int64_t m, double rho, WqPlan &p) {
    memset(&p, 0, sizeof(p));
    if (n < 2 || d < 1 || m < 1) return RMM_ERR_INVALID_ARG;
    p.k = k_of(rho, d);
    if (p.k < 1) return RMM_ERR_INVALID_ARG;
    if (n % 8 || d % 8 || m % 16 || d >= 0xffff || n > INT32_MAX / 2 || m > INT32_MAX / 2 ||
        n * d * 2 >= kMaxBufferBytes)
        return RMM_ERR_UNSUPPORTED;
    p.kpad = (p.k + 127) / 128 * 128;
    p.gc = gemm_choose_transposed(n, m, p.k, d);
    if (p.gc.tile != 5) {
        // few tiles or few K steps: the same kernel, its K range split as the chooser asks
        p.gc.tile = 5;
        if (p.gc.splits < 1) p.gc.splits = 1;
    }
    while (!gemm_tdma_fits(p.kpad, p.gc.splits, d, 1) && p.gc.splits < 64) ++p.gc.splits;
    if (!gemm_tdma_fits(p.kpad, p.gc.splits, d, 1)) return RMM_ERR_UNSUPPORTED;
    p.cp = colnorm_transpose_plan(n, d);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align_up(bytes);
        return o;
    };
    p.off_part = take((size_t)p.cp.chunks * d * 4);
    p.off_s = take((size_t)d * 4);
    p.off_idx = take((size_t)p.kpad * 4);
    p.off_At = take((size_t)d * n * 2);
    if (p.gc.splits > 1) p.off_gpart = take((size_t)p.gc.splits * n * m * 4);
    p.total = off;
    return RMM_OK;
}
}  // namespace
}  // namespace rmm

extern "C" size_t rmm_matmul_wq_workspace_size(int64_t n, int64_t d, int64_t m, double rho) {
    if (n == 1) return rmm_decode_wq_workspace_size(d, m, rho);
    WqPlan p;
    return wq_plan(n, d, m, rho, p) == RMM_OK ? p.total : SIZE_MAX;
}

extern "C" rmm_status_t rmm_matmul_wq(const void *A, int64_t n, int64_t d, int64_t lda, const void *Bq, int32_t fmt,
                                      const float *scale, int64_t m, int64_t ldb, double rho, float alpha, void *Y,
                                      int64_t ldy, int32_t *idx_out, void *workspace, size_t ws_bytes,
                                      hipStream_t stream) {
    if (!A || !Bq || !scale || !Y || (fmt != RMM_WQ_FP8_E4M3 && fmt != RMM_WQ_INT8) || n < 1 || d < 1 || m < 1 ||
        lda < d || ldb < m || ldy < m || !isfinite(alpha))
        return RMM_ERR_INVALID_ARG;
    if (n == 1)  // a single row: the decode route (ranking |a_j|, the gathered 8-bit GEMV)
        return rmm_decode_wq(A, Bq, fmt, scale, d, m, ldb, rho, alpha, Y, idx_out, workspace, ws_bytes, stream);
    WqPlan p;
    rmm_status_t st = wq_plan(n, d, m, rho, p);
    if (st != RMM_OK) return st;
    const int64_t ab = ((n - 1) * lda + d) * 2, bb = (d - 1) * ldb + m, sb = m * 4, yb = ((n - 1) * ldy + m) * 2;
    if (lda % 8 || ldy % 8 || ldb % 16 || !aligned16(A) || !aligned16(Bq) || !aligned16(Y) || !aligned16(scale) ||
        ab >= kMaxBufferBytes || bb >= kMaxBufferBytes)
        return RMM_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < p.total) return RMM_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255) return RMM_ERR_INVALID_ARG;
    char *ws = static_cast<char *>(workspace);
    const int64_t wb = (int64_t)p.total;
    if (overlaps(Y, yb, A, ab) || overlaps(Y, yb, Bq, bb) || overlaps(Y, yb, scale, sb) || overlaps(ws, wb, A, ab) ||
        overlaps(ws, wb, Bq, bb) || overlaps(ws, wb, scale, sb) || overlaps(ws, wb, Y, yb) ||
        (idx_out && (overlaps(idx_out, p.k * 4, Y, yb) || overlaps(idx_out, p.k * 4, ws, wb) ||
                     overlaps(idx_out, p.k * 4, A, ab) || overlaps(idx_out, p.k * 4, Bq, bb))))
        return RMM_ERR_INVALID_ARG;
    float *part = reinterpret_cast<float *>(ws + p.off_part);
    float *s = reinterpret_cast<float *>(ws + p.off_s);
    int32_t *pidx = reinterpret_cast<int32_t *>(ws + p.off_idx);
    uint16_t *At = reinterpret_cast<uint16_t *>(ws + p.off_At);
    // steps 1-2 on A alone (the set does not depend on the weights), A^T for the row gathers
    RMM_LAUNCH(RMM_KERNEL_COLNORM, launch_colnorm_transpose(A, n, d, lda, p.cp, At, n, part, stream));
    if (norm_select_ok(p.cp.chunks, d)) {
        RMM_LAUNCH(RMM_KERNEL_SELECT, launch_norm_select(part, p.cp.chunks, d, 1, p.k, idx_out, p.k, pidx, p.kpad,
                                                         stream));
    } else {
        RMM_LAUNCH(RMM_KERNEL_FINALIZE, launch_colnorm_finalize(part, p.cp.chunks, d, 1, s, stream));
        RMM_LAUNCH(RMM_KERNEL_SELECT,
                   launch_select(s, nullptr, RMM_F32, 0, 1, d, p.k, idx_out, p.k, pidx, p.kpad, nullptr, stream));
    }
    // steps 3-4: kept rows of A^T and of the codes, widened to bf16 in the kernel, scaled per column
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A = At;
    g.lda = n;
    g.a_bytes = d * n * 2;
    g.B = static_cast<const uint16_t *>(Bq);
    g.ldb = ldb;
    g.b_bytes = bb;
    g.group = 1;
    g.bmode = 0;
    g.idx = pidx;
    g.ld_idx = p.kpad;
    g.Y = static_cast<uint16_t *>(Y);
    g.ldy = ldy;
    g.n = n;
    g.m = m;
    g.k = p.k;
    g.kpad = p.kpad;
    g.batch = 1;
    g.alpha = alpha;
    g.splits = p.gc.splits;
    g.part = p.gc.splits > 1 ? reinterpret_cast<float *>(ws + p.off_gpart) : nullptr;
    g.bq = fmt == RMM_WQ_FP8_E4M3 ? 1 : 2;
    g.colscale = scale;
    RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_bf16(g, p.gc, stream));
    if (p.gc.splits > 1)  // the partials already carry the column scales
        RMM_LAUNCH(RMM_KERNEL_REDUCE, launch_splitk_reduce(g.part, p.gc.splits, n, m, 1, alpha,
                                                           static_cast<uint16_t *>(Y), ldy, 0, stream));
    return RMM_OK;
}

// ---------------------------------------------------------------- entry point without allocations
// rmm_matmul_noalloc takes its workspace from this array instead of the
// caller: one copy per GPU, alive until the process ends.  In host code the
// name `scratch` is only a host-side stand-in, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[RMM_NOALLOC_SCRATCH_BYTES];

namespace rmm {
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

// Device address of the current device's scratch array (resolved on the
// first call on that device).
rmm_status_t scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_error = e;
        return RMM_ERR_HIP;
    }
    if (dev < 0 || dev >= kScratchDevices) return RMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_error = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return RMM_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RMM_OK;
}
}  // namespace
}  // namespace rmm

extern "C" rmm_status_t rmm_matmul_noalloc(const rmm_desc_t *desc, const void *A, const void *B, double rho, void *Y,
                                           int32_t *idx_out, hipStream_t stream) {
    int64_t extA, extB, extY;
    rmm_status_t st = check_desc(desc, extA, extB, extY);
    if (st != RMM_OK) return st;
    if (!A || !B || !Y) return RMM_ERR_INVALID_ARG;
    const int64_t k = k_of(rho, desc->d);
    if (k < 1) return RMM_ERR_INVALID_ARG;
    // the plan for these very pointers (their alignment picks the route) must fit the array
    if (make_plan(desc, k, A, B, Y).total > (size_t)RMM_NOALLOC_SCRATCH_BYTES) return RMM_ERR_WORKSPACE;
    void *ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != RMM_OK) return st;
    return run_matmul(desc, A, B, k, nullptr, Y, idx_out, ws, (size_t)RMM_NOALLOC_SCRATCH_BYTES, stream, extA, extB,
                      extY);
}

namespace rmm {

namespace {

// Steps 1-4 of rmm_matmul once the arguments are known to be valid; with
// idx_in (rmm_matmul_indexed) the kept set is the caller's instead of steps
// 1-2.
rmm_status_t run_matmul(const rmm_desc_t *desc, const void *A, const void *B, int64_t k, const int32_t *idx_in,
                        void *Y, int32_t *idx_out, void *workspace, size_t ws_bytes, hipStream_t stream,
                        int64_t extA, int64_t extB, int64_t extY) {
    const rmm_desc_t &ds = *desc;
    const int64_t esz = ds.dtype == RMM_BF16 ? 2 : 4;
    if (overlaps(Y, extY * esz, A, extA * esz) || overlaps(Y, extY * esz, B, extB * esz)) return RMM_ERR_INVALID_ARG;
    if (idx_out && (overlaps(idx_out, k * ds.batch * 4, Y, extY * esz) ||
                    overlaps(idx_out, k * ds.batch * 4, A, extA * esz) ||
                    overlaps(idx_out, k * ds.batch * 4, B, extB * esz)))
        return RMM_ERR_INVALID_ARG;
    if (idx_in && overlaps(idx_in, k * ds.batch * 4, Y, extY * esz)) return RMM_ERR_INVALID_ARG;

    const Plan p = make_plan(desc, k, A, B, Y, idx_in != nullptr);
    if (p.total > 0 && (!workspace || ws_bytes < p.total)) return RMM_ERR_WORKSPACE;
    if (p.total > 0 && ((uintptr_t)workspace & 255)) return RMM_ERR_INVALID_ARG;  // pieces are 256-byte aligned
    char *ws = static_cast<char *>(workspace);
    if (p.total > 0 && (overlaps(ws, (int64_t)p.total, Y, extY * esz) || overlaps(ws, (int64_t)p.total, A, extA * esz) ||
                        overlaps(ws, (int64_t)p.total, B, extB * esz) ||
                        (idx_in && overlaps(ws, (int64_t)p.total, idx_in, k * ds.batch * 4))))
        return RMM_ERR_INVALID_ARG;

    const int64_t n = ds.n, d = ds.d, m = ds.m, batch = ds.batch;
    int32_t *pidx = reinterpret_cast<int32_t *>(ws + p.off_idx);  // padded: kpad per row

    if (p.fused_decode) {
        float *gpart = reinterpret_cast<float *>(ws + p.off_gpart);
        RMM_LAUNCH(RMM_KERNEL_GEMV, launch_decode_fused(static_cast<const uint16_t *>(A), d, k, B, 0, ds.ldb, m, nullptr,
                                                        ds.alpha, static_cast<uint16_t *>(Y), idx_out, p.gsplits,
                                                        gpart, stream));
        if (p.gsplits > 1)
            RMM_LAUNCH(RMM_KERNEL_REDUCE, launch_splitk_reduce(gpart, p.gsplits, 1, m, 1, ds.alpha,
                                                               static_cast<uint16_t *>(Y), ds.ldy, 0, stream));
        return RMM_OK;
    }
    if (p.route == ROUTE_DECODE) {
        float *aval = reinterpret_cast<float *>(ws + p.off_aval);
        float *gpart = reinterpret_cast<float *>(ws + p.off_gpart);
        if (idx_in)
            RMM_LAUNCH(RMM_KERNEL_SELECT, launch_index_prepare(idx_in, 1, k, d, pidx, p.kpad, A, aval, stream));
        else
            RMM_LAUNCH(RMM_KERNEL_SELECT,
                       launch_select(nullptr, A, RMM_BF16, 0, 1, d, k, idx_out, k, pidx, p.kpad, aval, stream));
        RMM_LAUNCH(RMM_KERNEL_GEMV, launch_gemv_partial(static_cast<const uint16_t *>(B), ds.ldb, m, pidx, aval, k,
                                                        p.gsplits, gpart, stream));
        RMM_LAUNCH(RMM_KERNEL_REDUCE, launch_splitk_reduce(gpart, p.gsplits, 1, m, 1, ds.alpha,
                                                           static_cast<uint16_t *>(Y), ds.ldy, 0, stream));
        return RMM_OK;
    }

    // steps 1-2: scores and selection (or every index at rho = 1)
    const int32_t *gemm_idx = pidx;
    if (idx_in) {
        RMM_LAUNCH(RMM_KERNEL_SELECT, launch_index_prepare(idx_in, batch, k, d, pidx, p.kpad, nullptr, nullptr, stream));
    } else if (p.shortcut) {
        if (idx_out) RMM_LAUNCH(RMM_KERNEL_OTHER, launch_iota(idx_out, k, k, batch, stream));
        gemm_idx = nullptr;  // identity
    } else {
        float *part = reinterpret_cast<float *>(ws + p.off_part);
        float *s = reinterpret_cast<float *>(ws + p.off_s);
        if (p.transA)
            RMM_LAUNCH(RMM_KERNEL_COLNORM, launch_colnorm_transpose(A, n, d, ds.lda, p.cp,
                                                                    reinterpret_cast<uint16_t *>(ws + p.off_At), n,
                                                                    part, stream));
        else
            RMM_LAUNCH(RMM_KERNEL_COLNORM,
                       launch_colnorm_partial(A, ds.dtype, n, d, ds.lda, batch, ds.strideA, p.cp, part, stream));
        if (norm_select_ok(p.cp.chunks, d)) {
            RMM_LAUNCH(RMM_KERNEL_SELECT, launch_norm_select(part, p.cp.chunks, d, batch, k, idx_out, k, pidx, p.kpad,
                                                             stream));
        } else {
            RMM_LAUNCH(RMM_KERNEL_FINALIZE, launch_colnorm_finalize(part, p.cp.chunks, d, batch, s, stream));
            RMM_LAUNCH(RMM_KERNEL_SELECT,
                       launch_select(s, nullptr, RMM_F32, 0, batch, d, k, idx_out, k, pidx, p.kpad, nullptr, stream));
        }
    }

    if (p.route == ROUTE_GENERIC) {
        GenericArgs g;
        g.dt = ds.dtype;
        g.A = A;
        g.lda = ds.lda;
        g.strideA = ds.strideA;
        g.B = B;
        g.ldb = ds.ldb;
        g.strideB = ds.strideB;
        g.group = ds.b_group;
        g.transB = ds.transB;
        g.idx = gemm_idx;
        g.ld_idx = p.kpad;
        g.Y = Y;
        g.ldy = ds.ldy;
        g.strideY = ds.strideY;
        g.n = n;
        g.m = m;
        g.k = k;
        g.batch = batch;
        g.alpha = ds.alpha;
        RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_generic(g, stream));
        return RMM_OK;
    }

    // ROUTE_MFMA: step 3 (gather) then step 4 (reduced product)
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    if (p.transA) {
        // both operands gathered by rows inside the GEMM: rows I_t of A^T and of B
        g.A = reinterpret_cast<const uint16_t *>(ws + p.off_At);
        g.lda = n;
        g.strideA = 0;
        g.a_bytes = d * n * 2;
        g.B = static_cast<const uint16_t *>(B);
        g.ldb = ds.ldb;
        g.strideB = 0;
        g.group = 1;
        g.bmode = 0;
        g.idx = pidx;
        g.ld_idx = p.kpad;
        g.Y = static_cast<uint16_t *>(Y);
        g.ldy = ds.ldy;
        g.strideY = 0;
        g.n = n;
        g.m = m;
        g.k = k;
        g.kpad = p.kpad;
        g.b_bytes = b_extent_bytes(desc);
        g.batch = 1;
        g.alpha = ds.alpha;
        g.splits = p.gc.splits;
        g.part = p.gc.splits > 1 ? reinterpret_cast<float *>(ws + p.off_gpart) : nullptr;
        RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_bf16(g, p.gc, stream));
        if (p.gc.splits > 1)
            RMM_LAUNCH(RMM_KERNEL_REDUCE, launch_splitk_reduce(g.part, p.gc.splits, n, m, 1, ds.alpha,
                                                               static_cast<uint16_t *>(Y), ds.ldy, 0, stream));
        return RMM_OK;
    }
    if (p.gc.tile == 6) {
        // A in place: the GEMM gathers the kept columns of 64-column windows itself
        if (!gemm_idx) {  // rho = 1 shortcut: every column, in order
            RMM_LAUNCH(RMM_KERNEL_OTHER, launch_iota(pidx, k, p.kpad, batch, stream));
            gemm_idx = pidx;
        }
        g.A = static_cast<const uint16_t *>(A);
        g.lda = ds.lda;
        g.strideA = ds.strideA;
        g.a_bytes = ((n - 1) * ds.lda + d) * 2;  // one entry: the last row ends at column d
        g.B = static_cast<const uint16_t *>(B);
        g.ldb = ds.ldb;
        g.strideB = ds.strideB;
        g.b_bytes = b_extent_bytes(desc);
        g.group = ds.b_group;
        g.bmode = 0;
        g.idx = gemm_idx;
        g.ld_idx = p.kpad;
        g.Y = static_cast<uint16_t *>(Y);
        g.ldy = ds.ldy;
        g.strideY = ds.strideY;
        g.n = n;
        g.m = m;
        g.k = k;
        g.kpad = p.kpad;
        g.batch = batch;
        g.alpha = ds.alpha;
        g.splits = 1;
        RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_bf16(g, p.gc, stream));
        return RMM_OK;
    }
    if (p.directA) {
        g.A = static_cast<const uint16_t *>(A);
        g.lda = ds.lda;
        g.strideA = ds.strideA;
    } else {
        uint16_t *Ap = reinterpret_cast<uint16_t *>(ws + p.off_Ap);
        if (p.shortcut) {
            // identity gather: the pack reads an index list; write 0..k-1 into the workspace one
            RMM_LAUNCH(RMM_KERNEL_OTHER, launch_iota(pidx, k, p.kpad, batch, stream));
            gemm_idx = pidx;
        }
        RMM_LAUNCH(RMM_KERNEL_PACK, launch_pack(A, RMM_BF16, n, d, ds.lda, ds.strideA, 1, pidx, p.kpad, p.kpad, Ap,
                                                p.a_rows * p.kpad, batch, p.gc.tile >= 2 ? 1 : 0, stream));
        g.A = Ap;
        g.lda = p.kpad;
        g.strideA = p.a_rows * p.kpad;
    }
    if (ds.transB) {
        uint16_t *Bp = reinterpret_cast<uint16_t *>(ws + p.off_Bp);
        if (!gemm_idx) {
            RMM_LAUNCH(RMM_KERNEL_OTHER, launch_iota(pidx, k, p.kpad, batch, stream));
            gemm_idx = pidx;
        }
        RMM_LAUNCH(RMM_KERNEL_PACK, launch_pack(B, RMM_BF16, m, d, ds.ldb, ds.strideB, ds.b_group, pidx, p.kpad,
                                                p.kpad, Bp, p.b_rows * p.kpad, batch, p.gc.tile == 3 ? 1 : 0,
                                                stream));
        g.B = Bp;
        g.ldb = p.kpad;
        g.strideB = p.b_rows * p.kpad;
        g.group = 1;
        g.bmode = 1;
        g.idx = nullptr;
    } else {
        if (!gemm_idx) {  // rho = 1 shortcut: the kernel reads rows 0..k-1 from the list
            RMM_LAUNCH(RMM_KERNEL_OTHER, launch_iota(pidx, k, p.kpad, batch, stream));
            gemm_idx = pidx;
        }
        g.B = static_cast<const uint16_t *>(B);
        g.ldb = ds.ldb;
        g.strideB = ds.strideB;
        g.group = ds.b_group;
        g.bmode = 0;
        g.idx = gemm_idx;
        g.ld_idx = p.kpad;
    }
    g.Y = static_cast<uint16_t *>(Y);
    g.ldy = ds.ldy;
    g.strideY = ds.strideY;
    g.n = n;
    g.m = m;
    g.k = k;
    g.kpad = p.directA ? d : p.kpad;
    g.a_bytes = p.directA ? a_extent_bytes(desc) : p.a_rows * p.kpad * 2;
    g.b_bytes = ds.transB ? p.b_rows * p.kpad * 2 : b_extent_bytes(desc);
    g.batch = batch;
    g.alpha = ds.alpha;
    g.splits = p.gc.splits;
    g.part = p.gc.splits > 1 ? reinterpret_cast<float *>(ws + p.off_gpart) : nullptr;
    RMM_LAUNCH(RMM_KERNEL_GEMM, launch_gemm_bf16(g, p.gc, stream));
    if (p.gc.splits > 1)
        RMM_LAUNCH(RMM_KERNEL_REDUCE, launch_splitk_reduce(g.part, p.gc.splits, n, m, batch, ds.alpha,
                                                           static_cast<uint16_t *>(Y), ds.ldy, ds.strideY, stream));
    return RMM_OK;
}

}  // namespace
}  // namespace rmm

extern "C" {

rmm_status_t rmm_timing_enable(int32_t enable, int32_t capacity) {
    TimingState &t = g_timing;
    if (!enable) {
        t.enabled = false;
        return RMM_OK;
    }
    if (capacity < 1 || capacity > (1 << 20)) return RMM_ERR_INVALID_ARG;
    if ((int)t.ev.size() < 2 * capacity) {
        for (size_t i = t.ev.size(); i < (size_t)2 * capacity; ++i) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return RMM_ERR_HIP;
            t.ev.push_back(e);
        }
    }
    t.kind.assign(capacity, 0);
    t.capacity = capacity;
    t.used = 0;
    t.enabled = true;
    return RMM_OK;
}

rmm_status_t rmm_timing_collect(double *ms, int64_t *count) {
    if (!ms || !count) return RMM_ERR_INVALID_ARG;
    for (int q = 0; q < RMM_KERNEL_KINDS; ++q) {
        ms[q] = 0.0;
        count[q] = 0;
    }
    TimingState &t = g_timing;
    for (int i = 0; i < t.used; ++i) {
        if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess) return RMM_ERR_HIP;
        float e = 0.f;
        if (hipEventElapsedTime(&e, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return RMM_ERR_HIP;
        ms[t.kind[i]] += e;
        count[t.kind[i]] += 1;
    }
    t.used = 0;
    return RMM_OK;
}

}  // extern "C"
