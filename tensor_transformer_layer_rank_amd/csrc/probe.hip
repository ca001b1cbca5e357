// Matrix-pipe rate microbenchmark: a measurement aid beside the shard computation, not part of
// it. Every wave issues v_mfma_f32_32x32x16_bf16 back to back on operands held in registers (no
// memory traffic inside the loop), 16 independent 32x32 accumulators per wave as in the GEMM
// tiles. With random operands the board's power limit sets the clock, and so the highest rate
// any bf16 GEMM can sustain on real data; low-entropy operands (zeros, ones) show the same
// pipe with little switching activity.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// ops: 8 fragments x 256 lanes x 16 bytes (fragments 0..3 are A operands, 4..7 B operands);
// out: one fp32 checksum per thread, so the accumulators stay live
__global__ __launch_bounds__(256, 1) void mfma_rate_kernel(const u32x4* __restrict__ ops, float* __restrict__ out,
                                                           int64_t iters) {
    const int tid = threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = __builtin_bit_cast(bf16x8, ops[i * 256 + tid]);
        b[i] = __builtin_bit_cast(bf16x8, ops[(4 + i) * 256 + tid]);
    }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][j][r];
    out[(int64_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace

hipError_t mfma_rate(const void* ops, float* out, int64_t n_wg, int64_t iters, hipStream_t s) {
    ProfScope ps("mfma_rate", s);
    mfma_rate_kernel<<<(unsigned)n_wg, 256, 0, s>>>(static_cast<const u32x4*>(ops), out, iters);
    return hipGetLastError();
}

}  // namespace tpk
