// Matrix-core throughput probe for measurement tools (rmm_calibrate_mfma).
//
// The reduced product's roofline is the bf16 matrix-core peak.  The
// datasheet figure (2.5 PFLOP/s dense bf16 on MI355X) assumes the top shader
// clock; under sustained matrix load the part runs power-limited below it.
// This kernel measures what the chip sustains: every wave issues
// v_mfma_f32_32x32x16_bf16 back to back on eight independent accumulators
// (no loads, no LDS, no dependence between consecutive instructions), so the
// only limit is the matrix pipe at whatever clock the chip holds.  The
// caller times the launch and divides the flops
//     workgroups * 4 waves * iters * 8 * (2 * 32 * 32 * 16)
// by the elapsed time.  The first wave of every workgroup also reads the
// shader-clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) around its loop, so the caller can tell the clock the
// chip held under this load: cycles / ticks * 100 MHz.
#include "rmm_internal.h"

namespace rmm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *__restrict__ out,
                                                        unsigned long long *__restrict__ clk) {
    // operands from the thread id so nothing is known at compile time; small
    // values keep every partial sum finite
    const uint32_t t = threadIdx.x + blockIdx.x * blockDim.x;
    const uint32_t bits = 0x3c003c00u ^ ((t & 7u) << 4) ^ ((t & 0x70u) << 16);
    const uint4 w = make_uint4(bits, bits ^ 0x10u, bits ^ 0x100000u, bits);
    bf16x8_t a = __builtin_bit_cast(bf16x8_t, w);
    bf16x8_t b = __builtin_bit_cast(bf16x8_t, make_uint4(w.y, w.z, w.w, w.x));
    f32x16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (clk && threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[t] = s;
}

}  // namespace
}  // namespace rmm

using namespace rmm;

extern "C" rmm_status_t rmm_calibrate_mfma(int64_t workgroups, int32_t iters, float *out, int64_t out_len,
                                           uint64_t *clk, hipStream_t stream) {
    if (!out || workgroups < 1 || workgroups > (1 << 20) || iters < 1 || out_len < workgroups * 256)
        return RMM_ERR_INVALID_ARG;
    mfma_peak_kernel<<<(unsigned)workgroups, 256, 0, stream>>>(iters, out,
                                                                reinterpret_cast<unsigned long long *>(clk));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? RMM_OK : RMM_ERR_HIP;
}
