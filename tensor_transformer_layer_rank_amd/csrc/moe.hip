// Top-k mixture-of-experts MLP on one rank ("TensorRT LLM 中的并行策略", 混合专家 (MoE): in
// the TP and hybrid ETP modes every local expert's weights are column/row split like a dense
// MLP shard, so each expert's rows produce partials and the gate-weighted combine, being
// linear, can run before the TP merge).
//
// Three steps on one stream: gather the dispatched rows (grouped by expert) from the token
// activations, run the experts' MLP shards on their rows (grouped GEMM launches across the
// experts, or the weight-streaming kernels expert by expert for small loads), and combine
// every token's rows, gate-weighted, in slot order. Row indices come from device
// arrays the host cannot see: an index outside its range contributes nothing (gathered
// row of zeros, skipped slot) instead of being dereferenced.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Xg[r, :] = X[row_token[r], :] (bf16, 16-byte chunks); one workgroup per row. Workgroups R and
// R + 1 (if launched) instead zero z.p[0] and z.p[1] (z.n[i] elements, multiples of 8): the zero
// rows that the grouped GEMMs' padding rows read.
struct ZeroRows {
    uint16_t* p[2];
    int64_t n[2];
};

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ X,
                                                          const int32_t* __restrict__ row_token,
                                                          uint16_t* __restrict__ Xg, int64_t R, int64_t T, int64_t H,
                                                          ZeroRows z) {
    const int64_t r = blockIdx.x;
    if (r >= R) {
        const int i = (int)(r - R);
        uint16_t* zp = i == 0 ? z.p[0] : z.p[1];
        const int64_t zn = i == 0 ? z.n[0] : z.n[1];
        for (int64_t c = threadIdx.x; c < (zn >> 3); c += 256)
            *reinterpret_cast<u32x4*>(zp + 8 * c) = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const int32_t t = row_token[r];
    const bool ok = t >= 0 && t < T;
    const int64_t nch = H >> 3;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
        const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(X + (int64_t)t * H + 8 * c) : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(Xg + r * H + 8 * c) = v;
    }
}

// Y[t, :] = sum_j gates[t, j] * Yg[token_rows[t, j], :] over the valid slots, in slot order
// (fp32); one workgroup per token
__global__ __launch_bounds__(256) void combine_rows_kernel(const float* __restrict__ Yg,
                                                           const int32_t* __restrict__ token_rows,
                                                           const float* __restrict__ gates, int k,
                                                           float* __restrict__ Y, int64_t R, int64_t H) {
    const int64_t t = blockIdx.x;
    const int64_t n4 = H >> 2;
    for (int64_t c = threadIdx.x; c < n4; c += 256) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int32_t r = token_rows[t * k + j];
            if (r < 0 || r >= R) continue;
            const float g = gates[t * k + j];
            acc += g * *reinterpret_cast<const f32x4*>(Yg + (int64_t)r * H + 4 * c);
        }
        *reinterpret_cast<f32x4*>(Y + t * H + 4 * c) = acc;
    }
}

}  // namespace

hipError_t moe_gather(const void* X, const int32_t* row_token, void* Xg, int64_t R, int64_t T, int64_t H,
                      hipStream_t s, void* z0, int64_t n0, void* z1, int64_t n1) {
    const ZeroRows z{{static_cast<uint16_t*>(z0), static_cast<uint16_t*>(z1)}, {z0 ? n0 : 0, z1 ? n1 : 0}};
    const int64_t blocks = R + (z0 || z1 ? 2 : 0);
    if (blocks == 0) return hipSuccess;
    ProfScope ps("moe_gather", s);
    gather_rows_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<const uint16_t*>(X), row_token,
                                                        static_cast<uint16_t*>(Xg), R, T, H, z);
    return hipGetLastError();
}

hipError_t moe_combine(const float* Yg, const int32_t* token_rows, const float* gates, int k, float* Y, int64_t T,
                       int64_t R, int64_t H, hipStream_t s) {
    ProfScope ps("moe_combine", s);
    combine_rows_kernel<<<(unsigned)T, 256, 0, s>>>(Yg, token_rows, gates, k, Y, R, H);
    return hipGetLastError();
}

}  // namespace tpk
