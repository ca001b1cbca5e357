// Backward of one rank's linear shard: dX = dY . W^T and dW = X^T . dY ("张量并行：切分
// Transformer 层的分布式训练", 列切分 / 行切分 and 前向与反向的通信对称: the same two products
// serve a column shard, whose dX is a partial the ranks sum, and a row shard, whose dX is the
// rank's complete slice; dW is local in both).
//
// Both products run on the bf16 MFMA GEMM, which takes its A operand K-contiguous and its B
// operand N-contiguous. W^T and X^T are therefore first written out transposed (bf16, an
// HBM-bound pass over W and X) into the caller's workspace; the GEMMs then read them in the
// layout they stream at full rate.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// out[C, R] = in[R, C]^T, bf16, R and C multiples of 8. One workgroup per 64 x 64 tile: 16-byte
// row chunks in, 16-byte chunks of the transposed rows out (8 consecutive lanes write 128
// contiguous bytes). In LDS, chunk c of tile row r sits at chunk position c ^ ((r >> 3) & 7),
// so the eight tile rows 8 apart that one output chunk gathers fall in different banks.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             uint16_t* __restrict__ out, int64_t R, int64_t C,
                                                             int64_t tiles_c) {
    __shared__ __attribute__((aligned(16))) uint16_t t[64 * 64];
    const int64_t ty = (int64_t)blockIdx.x / tiles_c, tx = (int64_t)blockIdx.x - ty * tiles_c;
    const int64_t r0 = ty * 64, c0 = tx * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int i = tid + p * 256;
        const int rr = i >> 3, cc = i & 7;
        if (r0 + rr < R && c0 + 8 * cc < C)
            *reinterpret_cast<u32x4*>(t + rr * 64 + 8 * (cc ^ ((rr >> 3) & 7))) =
                *reinterpret_cast<const u32x4*>(in + (r0 + rr) * C + c0 + 8 * cc);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int i = tid + p * 256;
        const int oc = i >> 3;          // output row in the tile = input column
        const int orr = (i & 7) * 8;    // output chunk = input rows orr .. orr+7
        if (c0 + oc < C && r0 + orr < R) {
            const int pc = (oc >> 3) ^ (orr >> 3);   // chunk position of column oc in rows orr..orr+7
            unsigned w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned lo = t[(orr + 2 * e) * 64 + 8 * pc + (oc & 7)];
                const unsigned hi = t[(orr + 2 * e + 1) * 64 + 8 * pc + (oc & 7)];
                w[e] = lo | (hi << 16);
            }
            *reinterpret_cast<u32x4*>(out + (c0 + oc) * R + r0 + orr) = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

hipError_t transpose_bf16(const void* in, void* out, int64_t R, int64_t C, hipStream_t s) {
    // 64x64 tiles of 256 threads: the caller keeps tiles below 2^24, so the grid's thread
    // count (tiles * 256) stays below 2^32
    const int64_t tiles_c = (C + 63) / 64, tiles = tiles_c * ((R + 63) / 64);
    ProfScope ps("transpose_bf16", s);
    transpose_bf16_kernel<<<(unsigned)tiles, 256, 0, s>>>(static_cast<const uint16_t*>(in),
                                                          static_cast<uint16_t*>(out), R, C, tiles_c);
    return hipGetLastError();
}

}  // namespace

size_t linear_backward_ws_bytes(int64_t T, int64_t K, int64_t N) {
    const size_t wt = (size_t)(N * K) * 2, xt = (size_t)(K * T) * 2;
    const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    if (N == T) return up(wt) + up(xt) + up(gemm_bf16_pair_split_bytes(T, K, K, N, N));
    const size_t a = gemm_bf16_split_bytes(T, K, N, 0), b = gemm_bf16_split_bytes(K, N, T, 0);
    return up(wt) + up(xt) + up(a > b ? a : b);
}

// dX [T, K] = dY [T, N] . W^T [N, K] and dW [K, N] = X^T [K, T] . dY [T, N]. When the two
// products share their inner size (N == T) they run as one launch, so the tail split fills
// the machine across both grids (two 176-tile grids on 256 units would each leave 80 idle).
hipError_t linear_backward(const void* X, const void* W, const void* dY, float* dX, float* dW, int64_t T,
                           int64_t K, int64_t N, void* ws, hipStream_t s) {
    const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    unsigned char* base = static_cast<unsigned char*>(ws);
    void* wt = base;                                   // W^T [N, K]
    void* xt = base + up((size_t)(N * K) * 2);         // X^T [K, T]
    unsigned char* split = static_cast<unsigned char*>(xt) + up((size_t)(K * T) * 2);
    const size_t split_bytes = linear_backward_ws_bytes(T, K, N) - (size_t)(split - base);
    hipError_t e = transpose_bf16(W, wt, K, N, s);
    if (e != hipSuccess) return e;
    if (N == T) {
        e = transpose_bf16(X, xt, T, K, s);
        if (e != hipSuccess) return e;
        return gemm_bf16_f32out_pair(dY, wt, dX, T, K, N, K, K, xt, dY, dW, K, N, T, N, N, N, split, split_bytes, s);
    }
    e = gemm_bf16_store(dY, wt, dX, T, K, N, N, K, K, 2, 0, split, split_bytes, s);
    if (e != hipSuccess) return e;
    e = transpose_bf16(X, xt, T, K, s);
    if (e != hipSuccess) return e;
    return gemm_bf16_store(xt, dY, dW, K, N, T, T, N, N, 2, 0, split, split_bytes, s);
}

}  // namespace tpk
