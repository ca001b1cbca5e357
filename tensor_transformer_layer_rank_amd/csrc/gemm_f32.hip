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

constexpr int TM = 64, TN = 64, TK = 16;   // block tile; 256 threads, 4x4 outputs each

template <bool RELU, bool ACCUM>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B,
                                                       float* __restrict__ C, int64_t M,
                                                       int64_t N, int64_t K, int64_t lda,
                                                       int64_t ldb, int64_t ldc) {
    __shared__ float As[TK][TM + 4];   // As[k][m]
    __shared__ float Bs[TK][TN + 4];   // Bs[k][n]
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;              // 16 x 16 threads, 4x4 outputs each
    const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
        // A tile TM x TK: 1024 values, 4 per thread
        for (int i = tid; i < TM * TK; i += 256) {
            const int mm = i / TK, kk = i % TK;
            const int64_t gm = m0 + mm, gk = k0 + kk;
            As[kk][mm] = (gm < M && gk < K) ? A[gm * lda + gk] : 0.0f;
        }
        for (int i = tid; i < TK * TN; i += 256) {
            const int kk = i / TN, nn = i % TN;
            const int64_t gk = k0 + kk, gn = n0 + nn;
            Bs[kk][nn] = (gk < K && gn < N) ? B[gk * ldb + gn] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gm = m0 + ty * 4 + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t gn = n0 + tx * 4 + j;
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

hipError_t gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, int64_t ldc, int relu, int accumulate,
                    hipStream_t s) {
    dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    ProfScope ps("gemm_f32", s);
    if (relu && accumulate)
        gemm_f32_kernel<true, true><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else if (relu)
        gemm_f32_kernel<true, false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else if (accumulate)
        gemm_f32_kernel<false, true><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    else
        gemm_f32_kernel<false, false><<<grid, 256, 0, s>>>(A, B, C, M, N, K, lda, ldb, ldc);
    return hipGetLastError();
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
