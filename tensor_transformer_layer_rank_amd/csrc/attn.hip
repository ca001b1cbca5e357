// Head-local causal flash attention for the prefill of a rank's attention shard
// ("CUDA tensor parallel computations", 放进 Transformer: once a head's Q, K and V are on
// the rank, Q_head K_head^T, softmax and the product with V_head are purely local;
// "张量并行：切分 Transformer 层的分布式训练", 自注意力块切分: scaled dot-product attention
// on the local heads). Grouped queries read kv head floor(j * hkv / hq)
// ("TensorRT LLM 中的并行策略", 注意力模块).
//
// Inputs are the QKV epilogue's head-major fp16 tensors: q [B, hq, S, 128],
// k [B, hkv, S, 128] and the transposed values vt [B, hkv, 128, S]. Output: bf16
// [B*S, hq*128], token-major, head h in columns h*128 .. h*128+127 (the rows of this rank's
// O shard).
//
// Work split: one workgroup = 4 wave64s = 128 consecutive queries of one (sequence, head);
// each wave owns 32 queries. Keys are visited in blocks of 64 up to the causal diagonal,
// double-buffered in LDS. The scores are formed transposed, S^T = K Q^T
// (v_mfma_f32_32x32x16_f16, keys = rows), so each lane holds 32 of the 64 scores of ONE
// query: the online-softmax max and sum need only the lane's own registers plus one
// exchange with the lane 32 apart. P^T stays in registers as the B operand of
// O^T += V^T P^T. Exponentials use exp2 with log2(e)/sqrt(128) folded into the scale.
// Query blocks are scheduled heaviest (longest causal prefix) first.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int QB = 128;          // queries per workgroup
constexpr int KB = 64;           // keys per block
constexpr int K_TILE = KB * 256; // 64 keys x 128 dims x 2 B
constexpr int V_TILE = 128 * KB * 2;
constexpr int STAGE = K_TILE + V_TILE;

// K tile: row = key (0..63), 16 chunks of 16 B per row
__device__ __forceinline__ int k_off(int row, int chunk) {
    return row * 256 + ((chunk ^ (row & 7)) << 4);
}
// V^T tile: row = dim (0..127), 8 chunks of 16 B (8 keys) per row
__device__ __forceinline__ int v_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row + (row >> 3)) & 7)) << 4);
}

struct KVRegs {
    u32x4 k[4];
    u32x4 v[4];
};

// K: 64 rows x 16 chunks = 1024 chunks, 4 per thread.
// V^T: 128 rows x 4 groups of 16 keys, 2 groups per thread (two 16-byte chunks each).
__device__ __forceinline__ void load_kv(KVRegs& r, const uint16_t* kp, const uint16_t* vp,
                                        int64_t S, int64_t key0, int tid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int q = tid + p * 256;
        const int row = q >> 4, c = q & 15;
        const int64_t key = key0 + row;
        r.k[p] = (key < S) ? *reinterpret_cast<const u32x4*>(kp + key * 128 + c * 8)
                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int u = tid + p * 256;
        const int d = u >> 2, grp = u & 3;
        const int64_t key = key0 + grp * 16;
        const uint16_t* src = vp + (int64_t)d * S + key;
        r.v[2 * p] = (key < S) ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
        r.v[2 * p + 1] = (key + 8 < S) ? *reinterpret_cast<const u32x4*>(src + 8)
                                       : u32x4{0u, 0u, 0u, 0u};
    }
}

// V^T chunk order inside each group of 16 keys: [k0..k3, k8..k11] [k4..k7, k12..k15], so that
// the MFMA lane half `hi` reads the 8 keys its P^T registers hold with one 16-byte load.
__device__ __forceinline__ void store_kv(const KVRegs& r, unsigned char* st, int tid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int q = tid + p * 256;
        *reinterpret_cast<u32x4*>(st + k_off(q >> 4, q & 15)) = r.k[p];
    }
    unsigned char* vs = st + K_TILE;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int u = tid + p * 256;
        const int d = u >> 2, grp = u & 3;
        const u32x4 a = r.v[2 * p], b = r.v[2 * p + 1];
        *reinterpret_cast<u32x4*>(vs + v_off(d, 2 * grp)) = u32x4{a.x, a.y, b.x, b.y};
        *reinterpret_cast<u32x4*>(vs + v_off(d, 2 * grp + 1)) = u32x4{a.z, a.w, b.z, b.w};
    }
}

__global__ __launch_bounds__(256, 2) void flash_attn_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ out,
                                                            int64_t S, int hq, int hkv, int B,
                                                            int nqb) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, hi = lane >> 5;
    const int bh_count = B * hq;
    const int qb = nqb - 1 - (int)(blockIdx.x / bh_count);   // heaviest first
    const int bh = (int)(blockIdx.x % bh_count);
    const int b = bh / hq, h = bh - b * hq;
    const int g = (h * hkv) / hq;
    const uint16_t* qp = q + ((int64_t)(b * hq + h) * S) * 128;
    const uint16_t* kp = k + ((int64_t)(b * hkv + g) * S) * 128;
    const uint16_t* vp = vt + ((int64_t)(b * hkv + g) * 128) * S;

    const int64_t q0 = (int64_t)qb * QB + wave * 32;   // first query of this wave
    const int64_t qrow = q0 + r32;                      // this lane's query
    f16x8 qf[8];
#pragma unroll
    for (int dk = 0; dk < 8; ++dk)
        qf[dk] = (qrow < S) ? __builtin_bit_cast(
                                  f16x8, *reinterpret_cast<const u32x4*>(qp + qrow * 128 + dk * 16 + hi * 8))
                            : f16x8{};

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;
    const float scale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

    int64_t kend = (int64_t)qb * QB + QB;
    if (kend > S) kend = S;
    const int nkb = (int)((kend + KB - 1) / KB);

    KVRegs regs;
    load_kv(regs, kp, vp, S, 0, tid);
    store_kv(regs, lds, tid);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const unsigned char* cur = lds + (kb & 1) * STAGE;
        unsigned char* nxt = lds + ((kb + 1) & 1) * STAGE;
        const bool more = kb + 1 < nkb;
        if (more) load_kv(regs, kp, vp, S, (int64_t)(kb + 1) * KB, tid);
        const int64_t key0 = (int64_t)kb * KB;
        if (key0 <= q0 + 31 && q0 < S) {   // some key of the block is visible to this wave
            f32x16 st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[t][r] = 0.0f;
#pragma unroll
                for (int dk = 0; dk < 8; ++dk) {
                    const f16x8 a = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const u32x4*>(cur + k_off(t * 32 + r32, dk * 2 + hi)));
                    st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[dk], st[t], 0, 0, 0);
                }
            }
            // scale, mask, block max over this query's 64 scores
            const bool diag = key0 + KB - 1 > q0;   // block reaches past some query of the wave
            float mblk = -__builtin_inff();
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float sv = st[t][r] * scale;
                    if (diag) {
                        const int64_t key = key0 + t * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        if (key > qrow || key >= S) sv = -__builtin_inff();
                    }
                    st[t][r] = sv;
                    mblk = fmaxf(mblk, sv);
                }
            mblk = fmaxf(mblk, __shfl_xor(mblk, 32));
            const float m_new = fmaxf(m_run, mblk);
            const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float lsum = 0.0f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(st[t][r] - m_use);
                    st[t][r] = p;
                    lsum += p;
                }
            lsum += __shfl_xor(lsum, 32);
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            // O^T += V^T P^T over 4 sub-blocks of 16 keys
            const unsigned char* vs = cur + K_TILE;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) pb[e] = (_Float16)st[ks >> 1][8 * (ks & 1) + e];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const f16x8 a = __builtin_bit_cast(
                        f16x8, *reinterpret_cast<const u32x4*>(vs + v_off(dt * 32 + r32, ks * 2 + hi)));
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb, o[dt], 0, 0, 0);
                }
            }
        }
        if (more) store_kv(regs, nxt, tid);
        __syncthreads();
    }
    if (qrow >= S) return;
    const float inv = 1.0f / l_run;
    const int64_t ld = (int64_t)hq * 128;
    uint16_t* op = out + ((int64_t)b * S + qrow) * ld + (int64_t)h * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d0 = dt * 32 + 8 * rq + 4 * hi;
            unsigned short w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(o[dt][4 * rq + e] * inv));
            const uint2 packed = make_uint2((unsigned)w[0] | ((unsigned)w[1] << 16),
                                            (unsigned)w[2] | ((unsigned)w[3] << 16));
            *reinterpret_cast<uint2*>(op + d0) = packed;
        }
}

}  // namespace

hipError_t flash_attn_fwd(const void* q, const void* k, const void* vt, void* out, int64_t B,
                          int64_t S, int hq, int hkv, hipStream_t s) {
    const int nqb = (int)((S + QB - 1) / QB);
    const int64_t blocks = (int64_t)nqb * B * hq;
    ProfScope ps("flash_attn_fwd", s);
    flash_attn_kernel<<<(unsigned)blocks, 256, 0, s>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(vt), static_cast<uint16_t*>(out), S, hq, hkv, (int)B, nqb);
    return hipGetLastError();
}

}  // namespace tpk
