// Exact fp32 path: LDS-tiled FMA GEMM for the column-parallel (optionally ReLU) and
// row-parallel (partial, optionally accumulating) linear layers, and the k-way partial
// sum ("CUDA tensor parallel computations": 第二类 Column Parallel, 第三类 Row Parallel,
// 第四类 all-reduce arithmetic).
//
// Each output is one fp32 FMA chain over k in increasing order. On integer-valued
// inputs whose partial sums stay below 2^24 every step is exact, so the result equals
// the exact product regardless of order.
#include "tp_internal.h"

namespace tpk {
namespace {

// Block tile of 16R x 16R outputs: 256 threads (16 x 16), R x R outputs each; R = 4 for
// larger products, R = 1 for small ones (more workgroups, a quarter of the FMA chain length
// per thread on the critical path). The 64-deep K tile fetches A and B of a K <= 64 product in
// one memory round trip (this path serves small, latency-bound layers).
constexpr int TK = 64;

template <int R, bool RELU, bool ACCUM>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ C, int64_t M,
                                                       int64_t N, int64_t K, int64_t lda,
                                                       int64_t ldb, int64_t ldc) {
    constexpr int TM = 16 * R, TN = 16 * R;
    constexpr int PER = TM * TK / 256;   // A (and B) values each thread loads per K tile
    static_assert(TM * TK % 256 == 0, "whole loads per thread");
    __shared__ float As[TK][TM + 4];   // As[k][m]
    __shared__ float Bs[TK][TN + 4];   // Bs[k][n]
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
    float acc[R][R] = {};
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        // A and B tiles, TM x TK and TK x TN: all of a thread's loads are issued before the
        // first is stored
        float av[PER], bv[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int i = tid + r * 256;
            const int64_t gm = m0 + i / TK, gk = k0 + i % TK;
            av[r] = (gm < M && gk < K) ? A[gm * lda + gk] : 0.0f;
            const int64_t hk = k0 + i / TN, hn = n0 + i % TN;
            bv[r] = (hk < K && hn < N) ? B[hk * ldb + hn] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int i = tid + r * 256;
            As[i % TK][i / TK] = av[r];
            Bs[i / TN][i % TN] = bv[r];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[R], b[R];
#pragma unroll
            for (int i = 0; i < R; ++i) a[i] = As[kk][ty * R + i];
#pragma unroll
            for (int j = 0; j < R; ++j) b[j] = Bs[kk][tx * R + j];
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < R; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t gm = m0 + ty * R + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t gn = n0 + tx * R + j;
            if (gn >= N) continue;
            float v = acc[i][j];
            if (RELU) v = v > 0.0f ? v : 0.0f;
            if (ACCUM) v += C[gm * ldc + gn];
            C[gm * ldc + gn] = v;
        }
    }
}

struct PartialPtrs {
    const float* p[16];
};

// out = ((p0 + p1) + p2) + ...; four floats per thread-step, then a scalar tail
__global__ __launch_bounds__(256) void partial_sum_kernel(PartialPtrs pk, int k,
                                                          float* __restrict__ out, int64_t n) {
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 acc = reinterpret_cast<const float4*>(pk.p[0])[i];
        for (int j = 1; j < k; ++j) {
            const float4 v = reinterpret_cast<const float4*>(pk.p[j])[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        reinterpret_cast<float4*>(out)[i] = acc;
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float acc = pk.p[0][i];
        for (int j = 1; j < k; ++j) acc += pk.p[j][i];
        out[i] = acc;
    }
}

}  // namespace

namespace {

template <int R>
hipError_t launch_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                      int64_t ldb, int64_t ldc, int relu, int accumulate, hipStream_t s) {
    constexpr int T = 16 * R;
    dim3 grid((unsigned)((N + T - 1) / T), (unsigned)((M + T - 1) / T));
    if (relu && accumulate)
        gemm_f32_kernel<R, true, true><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else if (relu)
        gemm_f32_kernel<R, true, false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else if (accumulate)
        gemm_f32_kernel<R, false, true><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else
        gemm_f32_kernel<R, false, false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    return hipGetLastError();
}

}  // namespace

// 64 x 64 tiles once they give the machine at least one workgroup per compute unit, 16 x 16
// tiles below that
hipError_t gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, int64_t ldc, int relu, int accumulate,
                    hipStream_t s) {
    ProfScope ps("gemm_f32", s);
    if (((M + 63) / 64) * ((N + 63) / 64) >= 256)
        return launch_f32<4>(A, B, C, M, N, K, lda, ldb, ldc, relu, accumulate, s);
    return launch_f32<1>(A, B, C, M, N, K, lda, ldb, ldc, relu, accumulate, s);
}

hipError_t partial_sum(const float* const* parts, int k, float* out, int64_t n, hipStream_t s) {
    PartialPtrs pk{};
    for (int i = 0; i < k; ++i) pk.p[i] = parts[i];
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    ProfScope ps("partial_sum", s);
    partial_sum_kernel<<<(unsigned)blocks, 256, 0, s>>>(pk, k, out, n);
    return hipGetLastError();
}

}  // namespace tpk
