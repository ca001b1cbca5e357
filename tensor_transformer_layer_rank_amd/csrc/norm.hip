// Residual add and RMS normalisation after the merge of a row-parallel block.
// "CUDA tensor parallel computations", 第四类 跨卡通信计算: the all-reduce turns the ranks'
// partial contributions into the block output; 第五类 局部逐元素计算: a norm reads a whole row
// of the hidden dimension, so it runs on that merged, replicated output. The step the next
// block needs: r = residual + sum of the partials, the new residual stream, and
// r / sqrt(mean(r^2) + eps) * gamma as its input (the usual RMSNorm; the pages give no
// formula).
//
// One workgroup (4 wave64s) per row, HBM-bound: each 16-byte chunk of every input is read
// once and each output chunk written once, with the row kept in registers between the sum
// of squares and the scaling. Inputs and outputs are streamed (nontemporal loads and stores)
// and, for 2, 4 or 8 partials, all of a chunk's loads are issued before the in-order adds
// (merge7b_tp4: 5.14 -> 5.56 TB/s). Thread t owns the 8-element chunks t, t + 256, ...; the sum of
// squares is reduced in a fixed order (per thread over its chunks, a fixed butterfly inside
// the wave, the four waves in order), so results are run-to-run identical.
#include <type_traits>

#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int NT = 256;

struct MergePtrs {
    const float* p[16];
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return (unsigned)__builtin_bit_cast(uint16_t, static_cast<__bf16>(a)) |
           ((unsigned)__builtin_bit_cast(uint16_t, static_cast<__bf16>(b)) << 16);
}

// C = chunks per thread (H / 8 <= 256 C). res_out may be res (each thread reads its chunks
// before the barrier and writes them after it).
// KC: the partial count when it is one of the common values (all loads of a chunk issued before
// the in-order adds), 0 for any other k (runtime loop).
template <int C, int KC>
__global__ __launch_bounds__(NT) void merge_rmsnorm_kernel(MergePtrs pk, int k, const uint16_t* res,
                                                           const uint16_t* __restrict__ gamma, float eps,
                                                           uint16_t* res_out, uint16_t* __restrict__ normed,
                                                           int64_t H) {
    __shared__ float wsum[NT / 64];
    const int tid = threadIdx.x;
    const int nch = (int)(H >> 3);
    const int64_t base = (int64_t)blockIdx.x * H;
    float r[C][8];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = tid + c * NT;
        if (ch < nch) {
            const int64_t off = base + (int64_t)ch * 8;
            f32x4 a0, a1;
            if constexpr (KC > 0) {
                f32x4 v0[KC], v1[KC];
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    v0[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pk.p[j] + off));
                    v1[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pk.p[j] + off + 4));
                }
                a0 = v0[0];
                a1 = v1[0];
#pragma unroll
                for (int j = 1; j < KC; ++j) {   // ((P0 + P1) + P2) + ...
                    a0 += v0[j];
                    a1 += v1[j];
                }
            } else {
                a0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pk.p[0] + off));
                a1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pk.p[0] + off + 4));
                for (int j = 1; j < k; ++j) {   // ((P0 + P1) + P2) + ...
                    a0 += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pk.p[j] + off));
                    a1 += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pk.p[j] + off + 4));
                }
            }
            const u32x4 rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(res + off));
            r[c][0] = bf16_lo(rv.x) + a0.x;
            r[c][1] = bf16_hi(rv.x) + a0.y;
            r[c][2] = bf16_lo(rv.y) + a0.z;
            r[c][3] = bf16_hi(rv.y) + a0.w;
            r[c][4] = bf16_lo(rv.z) + a1.x;
            r[c][5] = bf16_hi(rv.z) + a1.y;
            r[c][6] = bf16_lo(rv.w) + a1.z;
            r[c][7] = bf16_hi(rv.w) + a1.w;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += r[c][e] * r[c][e];
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if ((tid & 63) == 0) wsum[tid >> 6] = ss;
    __syncthreads();
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = tid + c * NT;
        if (ch < nch) {
            const int64_t off = base + (int64_t)ch * 8;
            const u32x4 gv = *reinterpret_cast<const u32x4*>(gamma + (int64_t)ch * 8);
            const float g[8] = {bf16_lo(gv.x), bf16_hi(gv.x), bf16_lo(gv.y), bf16_hi(gv.y),
                                bf16_lo(gv.z), bf16_hi(gv.z), bf16_lo(gv.w), bf16_hi(gv.w)};
            u32x4 ro, no;
            ro.x = pack_bf16(r[c][0], r[c][1]);
            ro.y = pack_bf16(r[c][2], r[c][3]);
            ro.z = pack_bf16(r[c][4], r[c][5]);
            ro.w = pack_bf16(r[c][6], r[c][7]);
            no.x = pack_bf16(r[c][0] * inv * g[0], r[c][1] * inv * g[1]);
            no.y = pack_bf16(r[c][2] * inv * g[2], r[c][3] * inv * g[3]);
            no.z = pack_bf16(r[c][4] * inv * g[4], r[c][5] * inv * g[5]);
            no.w = pack_bf16(r[c][6] * inv * g[6], r[c][7] * inv * g[7]);
            __builtin_nontemporal_store(ro, reinterpret_cast<u32x4*>(res_out + off));
            __builtin_nontemporal_store(no, reinterpret_cast<u32x4*>(normed + off));
        }
    }
}

}  // namespace

hipError_t merge_rmsnorm(const float* const* parts, int k, const void* residual, const void* gamma, float eps,
                         void* residual_out, void* normed, int64_t T, int64_t H, hipStream_t s) {
    MergePtrs pk{};
    for (int i = 0; i < k; ++i) pk.p[i] = parts[i];
    const int nch = (int)(H / 8);
    const auto* res = static_cast<const uint16_t*>(residual);
    const auto* g = static_cast<const uint16_t*>(gamma);
    auto* ro = static_cast<uint16_t*>(residual_out);
    auto* no = static_cast<uint16_t*>(normed);
    ProfScope ps("merge_rmsnorm", s);
    const dim3 grid((unsigned)T);
    auto go = [&](auto kc_t) {
        constexpr int KC = decltype(kc_t)::value;
        if (nch <= NT) merge_rmsnorm_kernel<1, KC><<<grid, NT, 0, s>>>(pk, k, res, g, eps, ro, no, H);
        else if (nch <= 2 * NT) merge_rmsnorm_kernel<2, KC><<<grid, NT, 0, s>>>(pk, k, res, g, eps, ro, no, H);
        else if (nch <= 4 * NT) merge_rmsnorm_kernel<4, KC><<<grid, NT, 0, s>>>(pk, k, res, g, eps, ro, no, H);
        else merge_rmsnorm_kernel<8, KC><<<grid, NT, 0, s>>>(pk, k, res, g, eps, ro, no, H);
    };
    if (k == 2) go(std::integral_constant<int, 2>{});
    else if (k == 4) go(std::integral_constant<int, 4>{});
    else if (k == 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 0>{});
    return hipGetLastError();
}

}  // namespace tpk
