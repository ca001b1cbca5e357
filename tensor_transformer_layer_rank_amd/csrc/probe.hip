// Measurement aids beside the shard computation, not part of it.
// Matrix-pipe rate microbenchmark. Every wave issues v_mfma_f32_32x32x16_bf16 back to back on operands held in registers (no
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

// HBM read rate at a decode GEMM's grid: workgroup w reads bytes [w * per_wg, (w + 1) * per_wg)
// of buf, its four waves taking the 8 KB blocks wave, wave + 4, ... with 16-byte nontemporal
// loads (8 per lane per block, the weight step of the decode GEMMs), the next block requested
// before the current one is folded in. 64 KB of LDS per workgroup holds the occupancy at two
// workgroups per compute unit, as in those GEMMs. out: one checksum per thread.
__global__ __launch_bounds__(256, 2) void hbm_read_kernel(const unsigned char* __restrict__ buf, int64_t per_wg,
                                                          unsigned* __restrict__ out) {
    __shared__ unsigned pad[16384];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned char* base = buf + (int64_t)blockIdx.x * per_wg;
    const int64_t nblk = per_wg / 8192;
    u32x4 acc = {0u, 0u, 0u, 0u}, cur[8], nxt[8];
    auto load = [&](u32x4 (&v)[8], int64_t blk) {   // blocks past the last re-read the last one
        const u32x4* p = reinterpret_cast<const u32x4*>(base + (blk < nblk ? blk : nblk - 1) * 8192) + lane;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(p + 64 * j);
    };
    load(cur, wave);
    for (int64_t b = wave; b < nblk; b += 4) {
        load(nxt, b + 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= cur[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) cur[j] = nxt[j];
    }
    pad[tid] = acc.x ^ acc.y;
    __syncthreads();
    out[(int64_t)blockIdx.x * 256 + tid] = acc.z ^ acc.w ^ pad[(tid + 1) & 255];
}

}  // namespace

hipError_t hbm_read(const void* buf, int64_t per_wg, int64_t n_wg, unsigned* out, hipStream_t s) {
    ProfScope ps("hbm_read", s);
    hbm_read_kernel<<<(unsigned)n_wg, 256, 0, s>>>(static_cast<const unsigned char*>(buf), per_wg, out);
    return hipGetLastError();
}

hipError_t mfma_rate(const void* ops, float* out, int64_t n_wg, int64_t iters, hipStream_t s) {
    ProfScope ps("mfma_rate", s);
    mfma_rate_kernel<<<(unsigned)n_wg, 256, 0, s>>>(static_cast<const u32x4*>(ops), out, iters);
    return hipGetLastError();
}

}  // namespace tpk
