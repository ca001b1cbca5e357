// Decode-step (one new token per sequence, M <= 64 rows) kernels of a rank's shard.
// The work is bound by streaming the weight shards and the KV cache from HBM once.
//
//   skinny_gemm_kernel   split-K GEMM A[M, K] . W[K, N] for small M: each wave streams a
//                        32 (k) x 128 (n) block of W per step with 128-bit loads (every byte
//                        of the weight read exactly once), transposes it in registers and
//                        feeds v_mfma_f32_16x16x32_bf16 with the activations as the A operand.
//                        The 4 waves of a workgroup take interleaved steps of one K chunk and
//                        are summed in LDS in a fixed order; chunks go to a partial buffer.
//   reduce kernels       sum the K-chunk partials in chunk order and apply the layer's
//                        epilogue: plain fp32/bf16 store (O and down partials, vocabulary-
//                        split logits), SiLU(gate)*up, or QKV: rotary embedding at the
//                        cache position, key/value append into the cache, q kept in fp32.
//   decode_attn_kernel   split-KV attention of one query over cache slots 0..L-1
//                        (16-lane groups read one 256-byte key row each), then a combine
//                        kernel merges the per-split (max, sum, output) triples.
//
// Sources: the column/row split of "CUDA tensor parallel computations" (第二类, 第三类), the
// attention shard of "放进 Transformer", and the KV cache kept per rank in
// "TensorRT LLM 中的并行策略" (注意力模块). The vocabulary-split output layer is from
// "张量并行：切分 Transformer 层的分布式训练" (输入与输出层).
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int STRIP = 128;   // output columns per workgroup
constexpr int STEP = 32;     // k rows per wave step (one MFMA depth)

struct SkinnyPlan {
    int64_t strips_per_b, strips, kchunk, splits, ncols;
};

SkinnyPlan plan_skinny(int64_t N, int64_t K, int nb) {
    SkinnyPlan p;
    p.strips_per_b = (N + STRIP - 1) / STRIP;
    p.strips = p.strips_per_b * nb;
    p.ncols = p.strips * STRIP;
    int64_t target = (768 + p.strips - 1) / p.strips;   // aim for ~768 workgroups
    if (target < 1) target = 1;
    int64_t kchunk = (K + target - 1) / target;
    kchunk = ((kchunk + 4 * STEP - 1) / (4 * STEP)) * (4 * STEP);   // whole steps for all 4 waves
    if (kchunk < 4 * STEP) kchunk = 4 * STEP;
    p.kchunk = kchunk;
    p.splits = (K + kchunk - 1) / kchunk;
    return p;
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <int MB>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(const uint16_t* __restrict__ A,
                                                          int64_t lda,
                                                          const uint16_t* __restrict__ B1,
                                                          const uint16_t* __restrict__ B2,
                                                          int64_t M, int64_t N, int64_t K,
                                                          int64_t kchunk, int64_t strips_per_b,
                                                          int64_t ncols, float* __restrict__ part) {
    __shared__ f32x4 red[4][MB * 16][STRIP / 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const int64_t strip = blockIdx.x, split = blockIdx.y;
    const uint16_t* Bp = (strip < strips_per_b) ? B1 : B2;
    const int64_t c0 = (strip % strips_per_b) * STRIP;
    const int64_t col = c0 + 8 * l16;
    const int64_t kbeg = split * kchunk;
    const int64_t kend = (kbeg + kchunk < K) ? kbeg + kchunk : K;
    const bool col_ok = col < N;

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t k0 = kbeg + wave * STEP; k0 < kend; k0 += 4 * STEP) {
        u32x4 w[8];
        const int64_t kr = k0 + 8 * grp;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = kr + i;
            w[i] = (row < kend && col_ok) ? *reinterpret_cast<const u32x4*>(Bp + row * N + col)
                                          : u32x4{0u, 0u, 0u, 0u};
        }
        bf16x8 a[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int64_t m = mb * 16 + l16;
            a[mb] = (m < M && kr < kend)
                        ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + m * lda + kr))
                        : bf16x8{};
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const unsigned sel = (t & 1) ? 0x07060302u : 0x05040100u;
            u32x4 bt;
            bt.x = __builtin_amdgcn_perm(w[1][t >> 1], w[0][t >> 1], sel);
            bt.y = __builtin_amdgcn_perm(w[3][t >> 1], w[2][t >> 1], sel);
            bt.z = __builtin_amdgcn_perm(w[5][t >> 1], w[4][t >> 1], sel);
            bt.w = __builtin_amdgcn_perm(w[7][t >> 1], w[6][t >> 1], sel);
            const bf16x8 b = __builtin_bit_cast(bf16x8, bt);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[mb][t], 0, 0, 0);
        }
    }
    // acc[mb][t][r] = C[m = mb*16 + 4*grp + r][col = c0 + 8*l16 + t]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + 4 * grp + r;
            red[wave][m][2 * l16] = f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            red[wave][m][2 * l16 + 1] = f32x4{acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
        }
    __syncthreads();
    for (int idx = tid; idx < MB * 16 * (STRIP / 4); idx += 256) {
        const int m = idx / (STRIP / 4), c4 = idx % (STRIP / 4);
        if (m >= M) continue;
        f32x4 s = red[0][m][c4];
        s += red[1][m][c4];
        s += red[2][m][c4];
        s += red[3][m][c4];
        *reinterpret_cast<f32x4*>(part + (split * M + m) * ncols + strip * STRIP + 4 * c4) = s;
    }
}

// out[m][n] = sum over splits (in order) of part[s][m][n]
__device__ __forceinline__ float sum_splits(const float* part, int splits, int64_t M,
                                            int64_t ncols, int64_t m, int64_t c) {
    float v = part[m * ncols + c];
    for (int s = 1; s < splits; ++s) v += part[((int64_t)s * M + m) * ncols + c];
    return v;
}

__global__ void reduce_store_kernel(const float* __restrict__ part, int splits, int64_t M,
                                    int64_t N, int64_t ncols, void* C, int64_t ldc, int kind) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx - m * N;
    const float v = sum_splits(part, splits, M, ncols, m, n);
    const int64_t off = m * ldc + n;
    if (kind == 0) static_cast<float*>(C)[off] = v;
    else if (kind == 1) static_cast<float*>(C)[off] += v;
    else if (kind == 2) static_cast<uint16_t*>(C)[off] = f32_to_bf16(v);
    else static_cast<uint16_t*>(C)[off] = f32_to_bf16(v > 0.f ? v : 0.f);
}

__global__ void reduce_swiglu_kernel(const float* __restrict__ part, int splits, int64_t M,
                                     int64_t I, int64_t ncols, int64_t up_off,
                                     uint16_t* __restrict__ h) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * I) return;
    const int64_t m = idx / I, c = idx - m * I;
    const float g = sum_splits(part, splits, M, ncols, m, c);
    const float u = sum_splits(part, splits, M, ncols, m, up_off + c);
    h[idx] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
}

// one thread per (sequence, head, i < 64); heads 0..hq-1 are q, then hkv k heads, then v
__global__ void reduce_qkv_decode_kernel(const float* __restrict__ part, int splits, int64_t B,
                                         int hq, int hkv, int64_t ncols, int64_t pos, double theta,
                                         float* __restrict__ qbuf, uint16_t* __restrict__ kc,
                                         uint16_t* __restrict__ vc, int64_t cap) {
    const int nh = hq + 2 * hkv;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * nh * 64) return;
    const int i = (int)(idx % 64);
    const int head = (int)((idx / 64) % nh);
    const int64_t b = idx / (64 * nh);
    const int64_t c = (int64_t)head * 128 + i;
    const float x1 = sum_splits(part, splits, B, ncols, b, c);
    const float x2 = sum_splits(part, splits, B, ncols, b, c + 64);
    if (head >= hq + hkv) {
        const int g = head - hq - hkv;
        uint16_t* dst = vc + ((b * hkv + g) * cap + pos) * 128;
        dst[i] = f32_to_bf16(x1);
        dst[i + 64] = f32_to_bf16(x2);
        return;
    }
    const double ang = (double)pos * pow(theta, -2.0 * (double)i / 128.0);
    const float cs = (float)cos(ang), sn = (float)sin(ang);
    const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
    if (head < hq) {
        float* dst = qbuf + (b * hq + head) * 128;
        dst[i] = y1;
        dst[i + 64] = y2;
    } else {
        const int g = head - hq;
        uint16_t* dst = kc + ((b * hkv + g) * cap + pos) * 128;
        dst[i] = f32_to_bf16(y1);
        dst[i + 64] = f32_to_bf16(y2);
    }
}

constexpr int CHUNK_MAX = 1024;

__device__ __forceinline__ float block_max(float v, float* sh) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}
__device__ __forceinline__ float block_sum(float v, float* sh) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

// grid (nsplit, hq, B); scratch[b][h][split][130] = (max in log2 units, sum, o[128])
__global__ __launch_bounds__(256) void decode_attn_kernel(const float* __restrict__ q,
                                                          const uint16_t* __restrict__ kc,
                                                          const uint16_t* __restrict__ vc,
                                                          int hq, int hkv, int64_t L, int64_t cap,
                                                          int64_t chunk, float* __restrict__ scratch) {
    __shared__ float sc[CHUNK_MAX];
    __shared__ float red[16][128];
    __shared__ float sh[4];
    const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
    const int split = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int g = (h * hkv) / hq;
    const int64_t kbeg = (int64_t)split * chunk;
    const int64_t kend = (kbeg + chunk < L) ? kbeg + chunk : L;
    const int n = (int)(kend - kbeg);
    const float scale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)
    float qv[8];
    const float* qp = q + (b * hq + h) * 128 + 8 * l16;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qp[e] * scale;
    const uint16_t* kb = kc + ((b * hkv + g) * cap) * 128 + 8 * l16;
    const uint16_t* vb = vc + ((b * hkv + g) * cap) * 128 + 8 * l16;
    for (int j = grp; j < n; j += 16) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(kb + (kbeg + j) * 128);
        float s = qv[0] * bf16_lo(kk.x) + qv[1] * bf16_hi(kk.x);
        s += qv[2] * bf16_lo(kk.y) + qv[3] * bf16_hi(kk.y);
        s += qv[4] * bf16_lo(kk.z) + qv[5] * bf16_hi(kk.z);
        s += qv[6] * bf16_lo(kk.w) + qv[7] * bf16_hi(kk.w);
        s += __shfl_xor(s, 8);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 1);
        if (l16 == 0) sc[j] = s;
    }
    __syncthreads();
    float mx = -__builtin_inff();
    for (int j = tid; j < n; j += 256) mx = fmaxf(mx, sc[j]);
    mx = block_max(mx, sh);
    float sm = 0.f;
    for (int j = tid; j < n; j += 256) {
        const float p = __builtin_amdgcn_exp2f(sc[j] - mx);
        sc[j] = p;
        sm += p;
    }
    sm = block_sum(sm, sh);   // its barriers also publish sc[]
    float acc[8] = {};
    for (int j = grp; j < n; j += 16) {
        const float p = sc[j];
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vb + (kbeg + j) * 128);
        acc[0] += p * bf16_lo(vv.x);
        acc[1] += p * bf16_hi(vv.x);
        acc[2] += p * bf16_lo(vv.y);
        acc[3] += p * bf16_hi(vv.y);
        acc[4] += p * bf16_lo(vv.z);
        acc[5] += p * bf16_hi(vv.z);
        acc[6] += p * bf16_lo(vv.w);
        acc[7] += p * bf16_hi(vv.w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[grp][8 * l16 + e] = acc[e];
    __syncthreads();
    float* dst = scratch + (((b * hq + h) * nsplit) + split) * 130;
    if (tid < 128) {
        float o = red[0][tid];
        for (int r = 1; r < 16; ++r) o += red[r][tid];
        dst[2 + tid] = o;
    }
    if (tid == 0) {
        dst[0] = mx;
        dst[1] = sm;
    }
}

// grid (hq, B), 128 threads: merge the splits of one (sequence, head) into bf16 output
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ scratch,
                                                             int nsplit, int hq,
                                                             uint16_t* __restrict__ out) {
    const int h = blockIdx.x, d = threadIdx.x;
    const int64_t b = blockIdx.y;
    const float* src = scratch + ((b * hq + h) * nsplit) * 130;
    float M = -__builtin_inff();
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, src[s * 130]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float w = __builtin_amdgcn_exp2f(src[s * 130] - M);
        num += w * src[s * 130 + 2 + d];
        den += w * src[s * 130 + 1];
    }
    out[(b * hq + h) * 128 + d] = f32_to_bf16(num / den);
}

int64_t decode_chunk(int64_t L, int* nsplit_out) {
    int64_t nsplit = 8;
    int64_t chunk = (L + nsplit - 1) / nsplit;
    chunk = ((chunk + 15) / 16) * 16;
    if (chunk > CHUNK_MAX) chunk = CHUNK_MAX;
    if (chunk < 16) chunk = 16;
    *nsplit_out = (int)((L + chunk - 1) / chunk);
    return chunk;
}

}  // namespace

size_t skinny_partials_bytes(int64_t M, int64_t N, int64_t K) {
    const SkinnyPlan p = plan_skinny(N, K, 1);
    return (size_t)(p.splits * M * p.ncols) * sizeof(float);
}

// B2 != nullptr: dual form; columns [0, ncols/2) come from B, [ncols/2, ncols) from B2
static hipError_t skinny_launch(const void* A, const void* B, const void* B2, float* part,
                                int64_t M, int64_t N, int64_t K, int64_t lda, int* splits_out,
                                int64_t* ncols_out, hipStream_t s, const char* name) {
    const SkinnyPlan p = plan_skinny(N, K, B2 ? 2 : 1);
    *splits_out = (int)p.splits;
    *ncols_out = p.ncols;
    dim3 grid((unsigned)p.strips, (unsigned)p.splits);
    const uint16_t* a = static_cast<const uint16_t*>(A);
    const uint16_t* b1 = static_cast<const uint16_t*>(B);
    const uint16_t* b2 = static_cast<const uint16_t*>(B2 ? B2 : B);
    ProfScope ps(name, s);
    if (M <= 32)
        skinny_gemm_kernel<2><<<grid, 256, 0, s>>>(a, lda, b1, b2, M, N, K, p.kchunk,
                                                   p.strips_per_b, p.ncols, part);
    else
        skinny_gemm_kernel<4><<<grid, 256, 0, s>>>(a, lda, b1, b2, M, N, K, p.kchunk,
                                                   p.strips_per_b, p.ncols, part);
    return hipGetLastError();
}

hipError_t skinny_gemm_partials(const void* A, const void* B, float* part, int64_t M, int64_t N,
                                int64_t K, int64_t lda, int* splits_out, hipStream_t s) {
    int64_t ncols;
    return skinny_launch(A, B, nullptr, part, M, N, K, lda, splits_out, &ncols, s, "skinny_gemm");
}

hipError_t skinny_reduce_store(const float* part, int splits, int64_t M, int64_t N, void* C,
                               int64_t ldc, int kind, hipStream_t s) {
    const SkinnyPlan p = plan_skinny(N, 1, 1);
    const int64_t n = M * N;
    ProfScope ps("skinny_reduce", s);
    reduce_store_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, splits, M, N, p.ncols,
                                                                    C, ldc, kind);
    return hipGetLastError();
}

// dual gate/up in one skinny launch, then SiLU(gate) * up into h
hipError_t skinny_swiglu(const void* X, const void* Wg, const void* Wu, float* part, void* h,
                         int64_t M, int64_t I, int64_t H, hipStream_t s) {
    int splits;
    int64_t ncols;
    hipError_t e = skinny_launch(X, Wg, Wu, part, M, I, H, H, &splits, &ncols, s, "skinny_gemm_gateup");
    if (e != hipSuccess) return e;
    const int64_t n = M * I;
    ProfScope ps("skinny_reduce_swiglu", s);
    reduce_swiglu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        part, splits, M, I, ncols, ncols / 2, static_cast<uint16_t*>(h));
    return hipGetLastError();
}

size_t skinny_swiglu_partials_bytes(int64_t M, int64_t I, int64_t H) {
    const SkinnyPlan p = plan_skinny(I, H, 2);
    return (size_t)(p.splits * M * p.ncols) * sizeof(float);
}

hipError_t skinny_reduce_qkv_decode(const float* part, int splits, int64_t B, int hq, int hkv,
                                    int64_t pos, float theta, float* qbuf, void* k_cache,
                                    void* v_cache, int64_t cap, hipStream_t s) {
    const int64_t N = (int64_t)(hq + 2 * hkv) * 128;
    const SkinnyPlan p = plan_skinny(N, 1, 1);
    const int64_t n = B * (hq + 2 * hkv) * 64;
    ProfScope ps("skinny_reduce_qkv", s);
    reduce_qkv_decode_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
        part, splits, B, hq, hkv, p.ncols, pos, (double)theta, qbuf,
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), cap);
    return hipGetLastError();
}

size_t decode_attn_scratch_bytes(int64_t B, int hq, int64_t L) {
    int nsplit;
    decode_chunk(L, &nsplit);
    return (size_t)(B * hq * nsplit * 130) * sizeof(float);
}

hipError_t decode_attn(const float* q, const void* k_cache, const void* v_cache, int64_t B,
                       int hq, int hkv, int64_t L, int64_t cap, float* scratch, void* out,
                       hipStream_t s) {
    int nsplit;
    const int64_t chunk = decode_chunk(L, &nsplit);
    {
        ProfScope ps("decode_attn", s);
        decode_attn_kernel<<<dim3((unsigned)nsplit, (unsigned)hq, (unsigned)B), 256, 0, s>>>(
            q, static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), hq,
            hkv, L, cap, chunk, scratch);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    ProfScope ps("decode_combine", s);
    decode_combine_kernel<<<dim3((unsigned)hq, (unsigned)B), 128, 0, s>>>(scratch, nsplit, hq,
                                                                        static_cast<uint16_t*>(out));
    return hipGetLastError();
}

}  // namespace tpk
