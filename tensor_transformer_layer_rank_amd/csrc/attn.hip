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
// Work split: one workgroup = 8 wave64s = 128 consecutive queries of one (sequence, head),
// one workgroup per compute unit (2 waves per SIMD). Keys are visited in blocks of 64 up to
// the causal diagonal; wave (slab, half) owns 32 queries and the 32 keys `half` of every
// block, and the two halves of a slab are merged once at the end (max, sum and output of two
// online softmaxes). The block loop is software-pipelined: the QK MFMAs of block kb+1 are
// issued while the VALU forms block kb's probabilities, with K one block ahead of V in the
// double-buffered LDS tiles. The grid (4 sequences x 8 heads x 16 query blocks
// = 512 for S = 2048) is twice the number of compute units and is dealt heaviest (longest
// causal prefix) first, so a unit that finishes a short block early takes the next longest:
// the causal triangle balances out across two rounds. The scores are formed transposed,
// S^T = K Q^T (v_mfma_f32_32x32x16_f16, keys = rows), so each lane holds 16 of the 32
// scores of ONE query: the online-softmax max and sum need only the lane's own registers
// plus one exchange with the lane 32 apart. P^T stays in registers as the B operand of
// O^T += V^T P^T. Exponentials use exp2 with log2(e)/sqrt(128) folded into the scale, and
// the exponent base of a query moves only when a block raises its maximum by more than 2^8
// (lazy rescaling), so the rescale of the accumulators is skipped on almost every block.
#include <type_traits>

#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int QB = 128;          // queries per workgroup
constexpr float TAU = 8.0f;      // lazy-rescale threshold (log2 units): probabilities <= 256
constexpr int NWAVE = 8;         // 4 query slabs x 2 key halves
constexpr int NT = NWAVE * 64;
constexpr int KB = 64;           // keys per block
constexpr int K_TILE = KB * 256; // 64 keys x 128 dims x 2 B
constexpr int V_TILE = 128 * KB * 2;
constexpr int STAGE = K_TILE + V_TILE;

// K tile: row = key (0..63), 16 chunks of 16 B per row; the chunk index is XOR-permuted
// by the row's low 4 bits, so the 16 rows that a quarter-wave reads (one chunk each) hit 16
// different 16-byte bank groups
__device__ __forceinline__ int k_off(int row, int chunk) {
    return row * 256 + ((chunk ^ (row & 15)) << 4);
}
// V^T tile: row = dim (0..127), 8 chunks of 16 B (8 keys) per row
__device__ __forceinline__ int v_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row + (row >> 3)) & 7)) << 4);
}

struct KVRegs {
    u32x4 k[2];
    u32x4 v[2];
};

// K: 64 rows x 16 chunks = 1024 chunks, 2 per thread.
// V^T: 128 rows x 4 groups of 16 keys, 1 group per thread (two 16-byte chunks).
// Keys past S are fetched from the last valid row / chunk instead (branch-free loads): their
// scores are masked to -inf, so their probabilities are exactly 0 and the finite stand-in
// values contribute nothing. S is a multiple of 8, so an 8-key chunk is wholly in or out.
__device__ __forceinline__ void load_k(KVRegs& r, const uint16_t* kp, int64_t S, int64_t key0, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int q = tid + p * NT;
        const int row = q >> 4, c = q & 15;
        const int64_t key = (key0 + row < S) ? key0 + row : S - 1;
        r.k[p] = *reinterpret_cast<const u32x4*>(kp + key * 128 + c * 8);
    }
}
__device__ __forceinline__ void load_v(KVRegs& r, const uint16_t* vp, int64_t S, int64_t key0, int tid) {
    const int d = tid >> 2, grp = tid & 3;
    const int64_t key = key0 + grp * 16;
    const int64_t k_lo = (key < S) ? key : S - 8;
    const int64_t k_hi = (key + 8 < S) ? key + 8 : S - 8;
    r.v[0] = *reinterpret_cast<const u32x4*>(vp + (int64_t)d * S + k_lo);
    r.v[1] = *reinterpret_cast<const u32x4*>(vp + (int64_t)d * S + k_hi);
}

__device__ __forceinline__ void store_k(const KVRegs& r, unsigned char* ks, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int q = tid + p * NT;
        *reinterpret_cast<u32x4*>(ks + k_off(q >> 4, q & 15)) = r.k[p];
    }
}
// V^T chunk order inside each group of 16 keys: [k0..k3, k8..k11] [k4..k7, k12..k15], so that
// the MFMA lane half `hi` reads the 8 keys its P^T registers hold with one 16-byte load.
__device__ __forceinline__ void store_v(const KVRegs& r, unsigned char* vs, int tid) {
    const int d = tid >> 2, grp = tid & 3;
    const u32x4 a = r.v[0], b = r.v[1];
    *reinterpret_cast<u32x4*>(vs + v_off(d, 2 * grp)) = u32x4{a.x, a.y, b.x, b.y};
    *reinterpret_cast<u32x4*>(vs + v_off(d, 2 * grp + 1)) = u32x4{a.z, a.w, b.z, b.w};
}

// S^T of one wave: its 32 keys (rows, from the K tile in LDS) x its 32 queries (qf), d = 128
__device__ __forceinline__ f32x16 qk_tile(const unsigned char* ks, const f16x8 (&qf)[8], int kh, int r32,
                                          int hi) {
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.0f;
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
        const f16x8 a0 = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(ks + k_off(kh * 32 + r32, dk * 2 + hi)));
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[dk], st, 0, 0, 0);
    }
    return st;
}

// -inf on the keys past the lane's query or past S (key0 = the wave's first key of the block)
__device__ __forceinline__ void mask_tile(f32x16& st, int64_t qrow, int64_t S, int64_t key0, int hi) {
    const int64_t lim64 = ((qrow < S - 1) ? qrow : S - 1) - key0;   // last visible key offset
    const int lim = (int)(lim64 < -1 ? -1 : (lim64 > 32 ? 32 : lim64));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * hi + (r & 3);
        st[r] = (kr > lim) ? -__builtin_inff() : st[r];
    }
}

constexpr int XCH_FLOATS = 66 * 64;   // (m, l, o[64 registers]) of one wave
constexpr int LDS_BYTES = (2 * STAGE > 4 * XCH_FLOATS * 4) ? 2 * STAGE : 4 * XCH_FLOATS * 4;

__global__ __launch_bounds__(NT, 1) void flash_attn_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ out,
                                                            int64_t S, int hq, int hkv, int B,
                                                            int nqb) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, hi = lane >> 5;
    const int slab = wave & 3, kh = wave >> 2;    // 32-query slab, 32-key half of each block
    const int bh_count = B * hq;
    const int qb = nqb - 1 - (int)(blockIdx.x / bh_count);   // heaviest first
    const int bh = (int)(blockIdx.x % bh_count);
    const int b = bh / hq, h = bh - b * hq;
    const int g = (h * hkv) / hq;
    const uint16_t* qp = q + ((int64_t)(b * hq + h) * S) * 128;
    const uint16_t* kp = k + ((int64_t)(b * hkv + g) * S) * 128;
    const uint16_t* vp = vt + ((int64_t)(b * hkv + g) * 128) * S;

    const int64_t q0 = (int64_t)qb * QB + slab * 32;   // first query of this wave
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

    // Software pipeline over key blocks: iteration kb issues the QK MFMAs of block kb+1 while
    // the VALU turns block kb's scores into probabilities, then multiplies them into O. K runs
    // one block ahead of V in LDS: iteration kb reads K tile kb+1 and V tile kb, and refills
    // the K buffer of block kb (with kb+2) and the V buffer of block kb-1 (with kb+1) from
    // registers loaded one iteration earlier (ra), while requesting K kb+3 and V kb+2 (rb).
    // Blocks past a wave's diagonal are computed fully masked (p = 0) rather than skipped, so
    // the pipeline has no data-dependent branches but the rare rescale.
    unsigned char* const kbuf0 = lds;
    unsigned char* const kbuf1 = lds + K_TILE;
    unsigned char* const vbuf0 = lds + 2 * K_TILE;
    unsigned char* const vbuf1 = lds + 2 * K_TILE + V_TILE;
    auto diag = [&](int blk) {   // some key of this wave's half of block blk is invisible
        const int64_t key0 = (int64_t)blk * KB + kh * 32;
        return key0 + 31 > q0 || key0 + 32 > S;
    };
    KVRegs ra, rb;
    load_k(ra, kp, S, 0, tid);
    load_v(ra, vp, S, 0, tid);
    store_k(ra, kbuf0, tid);
    store_v(ra, vbuf0, tid);
    if (nkb > 1) {
        load_k(ra, kp, S, KB, tid);
        store_k(ra, kbuf1, tid);
        load_v(ra, vp, S, KB, tid);
    }
    if (nkb > 2) load_k(ra, kp, S, 2 * KB, tid);
    __syncthreads();
    f32x16 s_cur = qk_tile(kbuf0, qf, kh, r32, hi);
    if (diag(0)) mask_tile(s_cur, qrow, S, (int64_t)kh * 32, hi);
    __syncthreads();   // every wave has read K tile 0 before iteration 0 refills its buffer
    // Steady iterations (the K and V of blocks kb+2, kb+3 exist and block kb+1 lies wholly
    // below this wave's diagonal) run a copy of the body without those checks; every wave
    // runs nkb iterations with one barrier each, whatever its split point.
    // The loop is unrolled by two so that the register sets (ra / rb) and the score tiles
    // (s_cur / s_nxt) swap roles by name instead of by copy, and the LDS buffer parity is a
    // compile-time constant.
    auto iteration = [&](int kb, auto steady_t, auto odd_t, KVRegs& ra, KVRegs& rb, f32x16& s_cur,
                         f32x16& s_nxt) {
        constexpr bool STEADY = decltype(steady_t)::value;
        constexpr bool odd = decltype(odd_t)::value;
        if (STEADY || kb + 3 < nkb) load_k(rb, kp, S, (int64_t)(kb + 3) * KB, tid);
        if (STEADY || kb + 2 < nkb) load_v(rb, vp, S, (int64_t)(kb + 2) * KB, tid);
        // block max of the raw scores; lazy rescaling: the exponent base m_run moves only
        // when some query's block maximum exceeds it by more than TAU (log2 units), so every
        // probability is at most 2^TAU (exact in fp16, no overflow in the fp32 sums) and the
        // rescale of l and the 64 accumulators runs only on the few blocks that raise a base.
        // The base cancels in the final division. -inf + TAU is -inf, so a query's first
        // visible key always sets its base.
        float mblk = s_cur[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mblk = fmaxf(mblk, s_cur[r]);
        mblk = fmaxf(mblk, __shfl_xor(mblk, 32)) * scale;   // scale > 0 keeps the order
        if (__ballot(mblk > m_run + TAU)) {
            const float m_new = fmaxf(m_run, mblk);
            const float alpha = (m_new == -__builtin_inff()) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -__builtin_inff()) ? 0.0f : m_run;   // all keys masked so far
        // next block's scores (MFMA) alongside this block's probabilities (VALU)
        s_nxt = qk_tile(odd ? kbuf0 : kbuf1, qf, kh, r32, hi);
        float lsum = 0.0f;
        f16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], scale, -m_use));
            lsum += pr;
            pb[r >> 3][r & 7] = (_Float16)pr;
        }
        // O^T += V^T P^T over this wave's two sub-blocks of 16 keys
        const unsigned char* vs = odd ? vbuf1 : vbuf0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const f16x8 a = __builtin_bit_cast(
                    f16x8, *reinterpret_cast<const u32x4*>(vs + v_off(dt * 32 + r32, (2 * kh + ks) * 2 + hi)));
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[ks], o[dt], 0, 0, 0);
            }
        lsum += __shfl_xor(lsum, 32);
        l_run += lsum;
        if (!STEADY && kb + 1 < nkb && diag(kb + 1))
            mask_tile(s_nxt, qrow, S, (int64_t)(kb + 1) * KB + kh * 32, hi);
        if (STEADY || kb + 2 < nkb) store_k(ra, odd ? kbuf1 : kbuf0, tid);
        if (STEADY || kb + 1 < nkb) store_v(ra, odd ? vbuf0 : vbuf1, tid);
        __syncthreads();
    };
    int steady_end = 0;
    while (steady_end + 3 < nkb && !diag(steady_end + 1)) ++steady_end;
    f32x16 s_nxt;
    for (int kb = 0; kb < nkb; kb += 2) {
        if (kb + 1 < steady_end) {
            iteration(kb, std::true_type{}, std::false_type{}, ra, rb, s_cur, s_nxt);
            iteration(kb + 1, std::true_type{}, std::true_type{}, rb, ra, s_nxt, s_cur);
        } else {
            iteration(kb, std::false_type{}, std::false_type{}, ra, rb, s_cur, s_nxt);
            if (kb + 1 < nkb) iteration(kb + 1, std::false_type{}, std::true_type{}, rb, ra, s_nxt, s_cur);
        }
    }
    // merge the two key halves of each slab: the kh = 1 wave hands (m, l, o) to the kh = 0 wave
    float* xch = reinterpret_cast<float*>(lds) + slab * XCH_FLOATS;
    if (kh == 1) {
        xch[lane] = m_run;
        xch[64 + lane] = l_run;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) xch[128 + (dt * 16 + r) * 64 + lane] = o[dt][r];
    }
    __syncthreads();
    if (kh == 1 || qrow >= S) return;
    const float m1 = xch[lane], l1 = xch[64 + lane];
    const float mm = fmaxf(m_run, m1);          // finite: key 0 is visible to every query
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    const float inv = 1.0f / (l_run * a0 + l1 * a1);
    const int64_t ld = (int64_t)hq * 128;
    uint16_t* op = out + ((int64_t)b * S + qrow) * ld + (int64_t)h * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d0 = dt * 32 + 8 * rq + 4 * hi;
            unsigned short w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * rq + e;
                const float v = (o[dt][r] * a0 + xch[128 + (dt * 16 + r) * 64 + lane] * a1) * inv;
                w[e] = __builtin_bit_cast(unsigned short, static_cast<__bf16>(v));
            }
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
    flash_attn_kernel<<<(unsigned)blocks, NT, 0, s>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(vt), static_cast<uint16_t*>(out), S, hq, hkv, (int)B, nqb);
    return hipGetLastError();
}

}  // namespace tpk
