// bf16 MFMA GEMM tiles for gfx950 (v_mfma_f32_32x32x16_bf16), used by every prefill-size
// linear layer of a rank's shard:
//   - column-parallel output, optional ReLU, bf16/fp16/fp32 store with a leading dimension
//     ("CUDA tensor parallel computations", 第二类 Column Parallel; 第五类 for the activation);
//   - row-parallel fp32 partial, overwrite or += (第三类 Row Parallel);
//   - gate/up dual GEMM with the SiLU(gate) * up epilogue: the two accumulators of a
//     column meet in the same lane and only h is stored ("张量并行：切分 Transformer 层的
//     分布式训练", MLP 块切分: gate and up multiplied element-wise, then down);
//   - fused QKV projection with the rotary embedding and a head-major scatter of Q, K
//     and V^T (自注意力块切分: each rank holds whole heads).
//
// Tile: 256 x 256 outputs per workgroup (gate/up: 256 rows x 128 h columns, i.e. 128
// gate + 128 up accumulator columns), K step 64, 512 threads = 8 wave64s laid out 4 (M)
// x 2 (N); each wave owns 64 x 128 outputs = 2 x 4 MFMA 32x32 blocks (128 fp32
// accumulators per lane).
// Staging: 128-bit global loads into registers one K step ahead; the weight block
// [K, N] (N contiguous in memory) is transposed in registers (v_perm) so that LDS holds
// both operands K-contiguous, which is what the MFMA operand layout wants (each lane
// supplies 8 consecutive k of one row/column). LDS is double buffered (2 x 64 KB) with an
// XOR swizzle of the 16-byte chunks so that the ds_read_b128 of 8 consecutive rows hit
// distinct banks.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 512;
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = BN * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;

// byte offset of 16-byte chunk `chunk` (0..7) of row `row` in a [rows][64] bf16 tile
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row + (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

struct GemmGeom {
    const uint16_t* A;    // [M, K] row-major, lda
    const uint16_t* B1;   // [K, N] row-major, ldb
    const uint16_t* B2;   // second weight of the dual (gate/up) form, else unused
    int64_t M, N, K, lda, ldb;
};

struct TileRegs {
    u32x4 a[4];
    u32x4 b[4];
};

template <bool DUAL>
__device__ __forceinline__ void load_tile(TileRegs& t, const GemmGeom& g, int64_t m0, int64_t n0,
                                          int64_t k0, int tid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int q = tid + p * NTHR;
        const int row = q >> 3, c = q & 7;
        const int64_t gm = m0 + row, gk = k0 + c * 8;
        if (gm < g.M && gk < g.K)
            t.a[p] = *reinterpret_cast<const u32x4*>(g.A + gm * g.lda + gk);
        else
            t.a[p] = u32x4{0u, 0u, 0u, 0u};
    }
    const int cg = tid & 31, rg = tid >> 5;
    const uint16_t* Bp;
    int64_t gn;
    if (DUAL) {
        Bp = (cg < 16) ? g.B1 : g.B2;
        gn = n0 + (int64_t)(cg & 15) * 8;
    } else {
        Bp = g.B1;
        gn = n0 + (int64_t)cg * 8;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gk = k0 + rg * 4 + i;
        if (gk < g.K && gn < g.N)
            t.b[i] = *reinterpret_cast<const u32x4*>(Bp + gk * g.ldb + gn);
        else
            t.b[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_tile(const TileRegs& t, unsigned char* stage, int tid) {
    unsigned char* As = stage;
    unsigned char* Bs = stage + A_BYTES;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int q = tid + p * NTHR;
        *reinterpret_cast<u32x4*>(As + lds_off(q >> 3, q & 7)) = t.a[p];
    }
    // this thread holds rows 4*rg..4*rg+3 (k) x columns 8*cg..8*cg+7 (n) of the weight
    // block; column c becomes 4 consecutive k of LDS row n = 8*cg + c.
    const int cg = tid & 31, rg = tid >> 5;
    const int kc = rg >> 1, half = rg & 1;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
        u32x2 v;
        v.x = __builtin_amdgcn_perm(t.b[1][c >> 1], t.b[0][c >> 1], sel);
        v.y = __builtin_amdgcn_perm(t.b[3][c >> 1], t.b[2][c >> 1], sel);
        const int n = cg * 8 + c;
        *reinterpret_cast<u32x2*>(Bs + lds_off(n, kc) + half * 8) = v;
    }
}

// LDS column (row of the transposed weight tile) of the j-th 32-wide block of wave wn
template <bool DUAL>
__device__ __forceinline__ int b_row_of(int j, int wn) {
    if (DUAL) return (j < 2) ? (wn * 64 + j * 32) : (128 + wn * 64 + (j - 2) * 32);
    return wn * 128 + j * 32;
}

template <bool DUAL>
__device__ __forceinline__ void compute_stage(f32x16 (&acc)[2][4], const unsigned char* stage,
                                              int wm, int wn, int lane) {
    const unsigned char* As = stage;
    const unsigned char* Bs = stage + A_BYTES;
    const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int chunk = ks * 2 + hi;
        bf16x8 a[2], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a[i] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(As + lds_off(wm * 64 + i * 32 + r32, chunk)));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(Bs + lds_off(b_row_of<DUAL>(j, wn) + r32, chunk)));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// row of accumulator register r of block i for a lane in half `hi` (MFMA 32x32 layout)
__device__ __forceinline__ int acc_row(int i, int r, int hi) {
    return i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
}

// ---- epilogues ----------------------------------------------------------------------

// KIND: 0 bf16, 1 fp16, 2 fp32 overwrite, 3 fp32 +=
template <int KIND, bool RELU>
struct EpiStore {
    void* C;
    int64_t ldc, M, N;
    __device__ void operator()(f32x16 (&acc)[2][4], int64_t m0, int64_t n0, int wm, int wn,
                               int lane) const {
        const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 128 + j * 32 + r32;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 64 + acc_row(i, r, hi);
                    if (row >= M) continue;
                    float v = acc[i][j][r];
                    if (RELU) v = v > 0.0f ? v : 0.0f;
                    const int64_t off = row * ldc + col;
                    if (KIND == 0) static_cast<uint16_t*>(C)[off] = f32_to_bf16(v);
                    else if (KIND == 1) static_cast<uint16_t*>(C)[off] = f32_to_f16(v);
                    else if (KIND == 2) static_cast<float*>(C)[off] = v;
                    else static_cast<float*>(C)[off] += v;
                }
        }
    }
};

struct EpiSwiGLU {
    uint16_t* h;   // [M, N] bf16
    int64_t M, N;
    __device__ void operator()(f32x16 (&acc)[2][4], int64_t m0, int64_t n0, int wm, int wn,
                               int lane) const {
        const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + r32;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 64 + acc_row(i, r, hi);
                    if (row >= M) continue;
                    const float gte = acc[i][j][r], up = acc[i][j + 2][r];
                    const float silu = gte / (1.0f + __expf(-gte));
                    h[row * N + col] = f32_to_bf16(silu * up);
                }
        }
    }
};

struct EpiQKV {
    QKVOut o;
    int64_t M;   // B*S
    __device__ void operator()(f32x16 (&acc)[2][4], int64_t m0, int64_t n0, int wm, int wn,
                               int lane) const {
        const int r32 = lane & 31, hi = lane >> 5;
        const int head = (int)((n0 + wn * 128) >> 7);   // one wave = one head of 128 columns
        const int n_heads = o.hq + 2 * o.hkv;
        if (head >= n_heads) return;
        const int64_t S = o.S;
        if (head < o.hq + o.hkv) {
            const bool is_q = head < o.hq;
            const int hh = is_q ? head : head - o.hq;
            const int nh = is_q ? o.hq : o.hkv;
            uint16_t* dst = static_cast<uint16_t*>(is_q ? o.q : o.k);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 64 + acc_row(i, r, hi);
                    if (row >= M) continue;
                    const int64_t b = row / S, s = row - b * S;
                    uint16_t* out = dst + ((b * nh + hh) * S + s) * 128;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int c = j * 32 + r32;               // pair (c, c + 64)
                        const float2 cs = o.rope[s * 64 + c];
                        const float x1 = acc[i][j][r], x2 = acc[i][j + 2][r];
                        out[c] = f32_to_f16(x1 * cs.x - x2 * cs.y);
                        out[c + 64] = f32_to_f16(x2 * cs.x + x1 * cs.y);
                    }
                }
        } else {
            const int hv = head - o.hq - o.hkv;
            uint16_t* vt = static_cast<uint16_t*>(o.vt);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 64 + acc_row(i, r, hi);
                    if (row >= M) continue;
                    const int64_t b = row / S, s = row - b * S;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int d = j * 32 + r32;
                        vt[((b * o.hkv + hv) * 128 + d) * S + s] = f32_to_f16(acc[i][j][r]);
                    }
                }
        }
    }
};

template <bool DUAL, class Epi>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(GemmGeom g, Epi epi, int tiles_m) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * (DUAL ? BN / 2 : BN);

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (int)((g.K + BK - 1) / BK);
    TileRegs t;
    load_tile<DUAL>(t, g, m0, n0, 0, tid);
    store_tile(t, smem, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        unsigned char* cur = smem + (kt & 1) * STAGE_BYTES;
        unsigned char* nxt = smem + ((kt + 1) & 1) * STAGE_BYTES;
        const bool more = kt + 1 < nk;
        if (more) load_tile<DUAL>(t, g, m0, n0, (int64_t)(kt + 1) * BK, tid);
        compute_stage<DUAL>(acc, cur, wm, wn, lane);
        if (more) store_tile(t, nxt, tid);
        __syncthreads();
    }
    epi(acc, m0, n0, wm, wn, lane);
}

template <bool DUAL, class Epi>
hipError_t launch(const GemmGeom& g, const Epi& epi, hipStream_t s, const char* name) {
    static bool attr_done[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 64 && !attr_done[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_kernel<DUAL, Epi>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_done[dev] = true;
    }
    const int64_t tiles_m = (g.M + BM - 1) / BM;
    const int64_t tiles_n = (g.N + (DUAL ? BN / 2 : BN) - 1) / (DUAL ? BN / 2 : BN);
    ProfScope ps(name, s);
    gemm_bf16_kernel<DUAL, Epi><<<(unsigned)(tiles_m * tiles_n), NTHR, LDS_BYTES, s>>>(g, epi, (int)tiles_m);
    return hipGetLastError();
}

__global__ void rope_table_kernel(float2* t, int64_t pos0, int64_t npos, double theta) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= npos * 64) return;
    const int64_t p = idx / 64;
    const int i = (int)(idx - p * 64);
    const double inv_freq = pow(theta, -2.0 * (double)i / 128.0);
    const double ang = (double)(pos0 + p) * inv_freq;
    t[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

}  // namespace

hipError_t gemm_bf16_store(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int out_kind,
                           int relu, hipStream_t s) {
    GemmGeom g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), nullptr,
               M, N, K, lda, ldb};
#define TP_STORE_CASE(KIND, RELU)                                                   \
    if (out_kind == KIND && (relu != 0) == RELU)                                    \
        return launch<false>(g, EpiStore<KIND, RELU>{C, ldc, M, N}, s,              \
                             KIND >= 2 ? "gemm_bf16_f32out" : "gemm_bf16_store");
    TP_STORE_CASE(0, false)
    TP_STORE_CASE(0, true)
    TP_STORE_CASE(1, false)
    TP_STORE_CASE(1, true)
    TP_STORE_CASE(2, false)
    TP_STORE_CASE(2, true)
    TP_STORE_CASE(3, false)
#undef TP_STORE_CASE
    return hipErrorInvalidValue;
}

hipError_t gemm_bf16_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                            int64_t N, int64_t K, hipStream_t s) {
    GemmGeom g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bg),
               static_cast<const uint16_t*>(Bu), M, N, K, K, N};
    return launch<true>(g, EpiSwiGLU{static_cast<uint16_t*>(h), M, N}, s, "gemm_bf16_swiglu");
}

hipError_t gemm_bf16_qkv_rope(const void* X, const void* Wqkv, int64_t H, const QKVOut& o,
                              hipStream_t s) {
    const int64_t M = o.B * o.S, N = (int64_t)(o.hq + 2 * o.hkv) * 128;
    GemmGeom g{static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wqkv), nullptr,
               M, N, H, H, N};
    return launch<false>(g, EpiQKV{o, M}, s, "gemm_bf16_qkv_rope");
}

hipError_t rope_table(float2* table, int64_t pos0, int64_t npos, float theta, hipStream_t s) {
    const int64_t n = npos * 64;
    ProfScope ps("rope_table", s);
    rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(table, pos0, npos, (double)theta);
    return hipGetLastError();
}

}  // namespace tpk
