// Head-local causal flash attention for the prefill of a rank's attention shard
// ("CUDA tensor parallel computations", 放进 Transformer: once a head's Q, K and V are on
// the rank, Q_head K_head^T, softmax and the product with V_head are purely local;
// "张量并行：切分 Transformer 层的分布式训练", 自注意力块切分: scaled dot-product attention
// on the local heads). Grouped queries read kv head floor(j * hkv / hq)
// ("TensorRT LLM 中的并行策略", 注意力模块).
//
// Inputs are the QKV epilogue's head-major fp16 tensors: q [B, hq, S, 128] (pre-multiplied
// by log2(e)/sqrt(128), so scores come out in log2 units), k [B, hkv, S, 128] and the
// transposed values vt [B, hkv, 128, S]. Output: bf16 [B*S, hq*128], token-major, head h in
// columns h*128 .. h*128+127 (the rows of this rank's O shard).
//
// Work split: one workgroup = 8 wave64s = 128 consecutive queries of one (sequence, head),
// one workgroup per compute unit (2 waves per SIMD). Keys are visited in blocks of 64 up to
// the causal diagonal; wave (slab, half) owns 32 queries and the 32 keys `half` of every
// block, and the two halves of a slab are merged once at the end (max, sum and output of two
// online softmaxes). K, V^T and the query tile reach LDS by DMA (global_load_lds, no register
// staging) through a ring of four 32 KB stages, two blocks ahead of use. The block loop is
// software-pipelined: the QK MFMAs of block kb+1 are issued while the VALU forms block kb's
// probabilities, then the PV MFMAs of block kb run; one barrier per block. The grid
// (4 sequences x 8 heads x 16 query blocks = 512 for S = 2048) is twice the number of compute
// units and is dealt heaviest (longest causal prefix) first, so a unit that finishes a short
// block early takes the next longest: the causal triangle balances out across two rounds.
// The scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_f16, keys = rows), so
// each lane holds 16 of the 32 scores of ONE query: the online-softmax max and sum need only
// the lane's own registers plus one exchange with the lane 32 apart (v_permlane32_swap). P^T
// stays in registers as the B operand of O^T += V^T P^T; the row sums are taken from the
// same fp16 probabilities (v_dot2_f32_f16). The exponent base of a query moves only when a
// block raises its maximum by more than 2^8 (lazy rescaling), so the rescale of the
// accumulators is skipped on almost every block.
#include <type_traits>

#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
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
constexpr int NSTAGE = 4;        // ring of key blocks in LDS: up to 2 blocks in flight ahead

// Rows of a K tile hold the keys of a block in the order that makes each lane's scores
// consecutive keys: within every 16 rows, bits 2 and 3 of the row index are swapped. The
// score accumulator of S^T = K Q^T puts rows 8j + 4 hi + (0..3) in a lane of half `hi`, so
// with this order the lane holds keys 16 (r >> 3) + 8 hi + (r & 7) in register r, i.e. the
// 8 consecutive keys per 16-key step that the B operand of O^T += V^T P^T wants, and V^T can
// be read as plain 8-key chunks. The order is applied by the DMA (source row per lane).
__device__ __forceinline__ int swap23(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// K tile: row = tile row (0..63), 16 chunks of 16 B per row; the chunk index is XOR-permuted
// by the row's low 4 bits, so the 16 rows that a quarter-wave reads (one chunk each) hit 16
// different 16-byte bank groups
__device__ __forceinline__ int k_off(int row, int chunk) {
    return row * 256 + ((chunk ^ (row & 15)) << 4);
}
// V^T tile: row = dim (0..127), 8 chunks of 16 B (8 keys) per row, XOR-permuted by a
// function of the row's low 5 bits (conflict-free reads of 32 consecutive rows; rows 32
// apart share the permutation, so the four 32-dim slices are immediate offsets apart)
__device__ __forceinline__ int v_swz(int row) { return ((row & 31) + ((row & 31) >> 3)) & 7; }
__device__ __forceinline__ int v_off(int row, int chunk) { return row * 128 + ((chunk ^ v_swz(row)) << 4); }

// One 16-byte global -> LDS transfer per lane from base + off (base wave-uniform); the lanes
// of a wave fill 64 consecutive granules starting at LDS address dst (wave-uniform). A
// volatile asm statement with no register outputs: the compiler neither reorders it against
// other memory accesses nor adds vmcnt waits for it; the kernel counts its own (4 transfers
// per thread and key block).
__device__ __forceinline__ void dma16(const void* base, unsigned off, unsigned dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(dst), "v"(off), "s"(base)
                 : "memory", "m0");
}

// vmcnt(N): at most N of this wave's vector memory operations outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Per-lane sources of this thread's 4 transfers of a key block: granule p = i * 512 +
// wave * 64 + lane of each tile (i = 0, 1), i.e. LDS byte p * 16 of the tile. Byte offsets
// from the block's first key (K: from row key0 of k; V^T: from column key0 of vt).
// S <= 2^24 keeps the V^T offsets (< 256 S bytes) in 32 bits.
struct KVSrc {
    unsigned k[2], v[2];
};

__device__ __forceinline__ KVSrc kv_src(int wave, int lane, int64_t S) {
    KVSrc r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int kr = i * 32 + wave * 4 + (lane >> 4);
        r.k[i] = (unsigned)(swap23(kr) * 256 + (((lane & 15) ^ (kr & 15)) << 4));
        const int d = i * 64 + wave * 8 + (lane >> 3);
        r.v[i] = (unsigned)(((int64_t)d * S + (((lane & 7) ^ v_swz(d)) << 3)) * 2);
    }
    return r;
}

// DMA key block blk (keys blk*64 ..) into a stage. Keys past S are fetched from the last
// valid row / chunk instead: their scores are masked to -inf, so their probabilities are
// exactly 0 and the finite stand-in values contribute nothing. S is a multiple of 8, so an
// 8-key chunk is wholly in or out.
__device__ __forceinline__ void issue_block(unsigned stage, const KVSrc& src, const uint16_t* kp,
                                            const uint16_t* vp, int64_t S, int blk, int wave, int lane) {
    const int64_t key0 = (int64_t)blk * KB;
    const uint16_t* kb = kp + key0 * 128;
    const uint16_t* vb = vp + key0;
    const unsigned kd = stage + wave * 1024;
    const unsigned vd = stage + K_TILE + wave * 1024;
    if (key0 + KB <= S) {
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(kb, src.k[i], kd + i * 8192);
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16(vb, src.v[i], vd + i * 8192);
        return;
    }
    const int last = (int)(S - 1 - key0);   // last valid key offset in the block (>= 0)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int kr = swap23(i * 32 + wave * 4 + (lane >> 4));
        const unsigned off = src.k[i] - kr * 256 + (kr < last ? kr : last) * 256;
        dma16(kb, off, kd + i * 8192);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int d = i * 64 + wave * 8 + (lane >> 3);
        const int c8 = ((lane & 7) ^ v_swz(d)) << 3;          // chunk's first key offset
        const int c8c = c8 <= last - 7 ? c8 : last - 7;        // last valid chunk (S % 8 == 0)
        dma16(vb, src.v[i] - c8 * 2 + c8c * 2, vd + i * 8192);
    }
}

// max / sum of a lane's value and the value of the lane 32 apart (v_permlane32_swap)
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// -inf on the keys past the lane's query or past S. q_lim = min(query, S-1) and key0 (the
// wave's first key of the block) are both relative to the workgroup's first query; register r
// holds key key0 + 16 (r >> 3) + 8 hi + (r & 7).
__device__ __forceinline__ void mask_tile(f32x16& st, int q_lim, int key0, int hi) {
    int lim = q_lim - key0;                  // last visible key offset
    lim = lim < -1 ? -1 : (lim > 32 ? 32 : lim);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kr = 16 * (r >> 3) + 8 * hi + (r & 7);
        st[r] = (kr > lim) ? -__builtin_inff() : st[r];
    }
}

constexpr int XCH_FLOATS = 66 * 64;   // (m, l, o[64 registers]) of one wave
constexpr int Q_TILE = QB * 256;      // the workgroup's queries, fp16, K-tile layout
constexpr int RING = (NSTAGE * STAGE > 4 * XCH_FLOATS * 4) ? NSTAGE * STAGE : 4 * XCH_FLOATS * 4;
constexpr int LDS_BYTES = RING + Q_TILE;
static_assert(LDS_BYTES <= 160 * 1024, "LDS of one compute unit");

__global__ __launch_bounds__(NT, 1) void flash_attn_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ vt,
                                                            uint16_t* __restrict__ out,
                                                            int64_t S, int hq, int hkv, int B,
                                                            int nqb) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int64_t qfirst = (int64_t)qb * QB;
    const int q_lim = (int)(((qrow < S - 1) ? qrow : S - 1) - qfirst);   // S <= 2^24: fits
    int64_t kend = (int64_t)qb * QB + QB;
    if (kend > S) kend = S;
    const int nkb = (int)((kend + KB - 1) / KB);

    // LDS address of the ring (wave-uniform)
    const unsigned lds_a = (unsigned)__builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)lds));
    // the query tile and the first three key blocks go out before anything else; query rows
    // past S are fetched from row S-1 (their outputs are not stored)
    {
        const int last = (int)(S - 1 - qfirst);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = i * 32 + wave * 4 + (lane >> 4);
            const int c = (lane & 15) ^ (row & 15);
            dma16(qp + qfirst * 128, (unsigned)(((row < last ? row : last) * 128 + c * 8) * 2),
                  lds_a + RING + i * 8192 + wave * 1024);
        }
    }
    const KVSrc src = kv_src(wave, lane, S);
    issue_block(lds_a, src, kp, vp, S, 0, wave, lane);
    if (nkb > 1) issue_block(lds_a + STAGE, src, kp, vp, S, 1, wave, lane);
    if (nkb > 2) issue_block(lds_a + 2 * STAGE, src, kp, vp, S, 2, wave, lane);
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;
    const f16x2 ones2 = {1, 1};

    // this lane's LDS read offsets inside a stage: 8 K fragments (one per 16-dim slice) and
    // the V^T fragments of its two 16-key sub-blocks (the four 32-dim slices are 4 KB apart)
    // K: row*256 + ((2 dk + hi) ^ (row & 15)) * 16 = k_rd0 + ((dk ^ k_x) << 5)
    const int k_row = kh * 32 + r32;
    const unsigned k_rd0 = (unsigned)(k_row * 256 + ((hi ^ (k_row & 1)) << 4));
    const unsigned k_x = (unsigned)((k_row >> 1) & 7);
    const unsigned v_rd0 = (unsigned)(K_TILE + v_off(r32, (2 * kh) * 2 + hi));
    const unsigned v_rd1 = (unsigned)(K_TILE + v_off(r32, (2 * kh + 1) * 2 + hi));
    auto k_frag = [&](const unsigned char* st, int dk) {
        return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(st + k_rd0 + (((unsigned)dk ^ k_x) << 5)));
    };
    auto v_frag = [&](const unsigned char* st, int ks, int dt) {
        return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(st + (ks ? v_rd1 : v_rd0) + dt * 4096));
    };
    auto diag = [&](int blk) {   // some key of this wave's half of block blk is invisible
        const int64_t key0 = (int64_t)blk * KB + kh * 32;
        return key0 + 31 > q0 || key0 + 32 > S;
    };
    auto stage_of = [&](int blk) { return lds + (blk & (NSTAGE - 1)) * STAGE; };

    // block 0's scores
    if (nkb > 2) wait_vm<8>();
    else if (nkb > 1) wait_vm<4>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    f16x8 qf[8];
#pragma unroll
    for (int dk = 0; dk < 8; ++dk)
        qf[dk] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(
                                               lds + RING + k_off(slab * 32 + r32, dk * 2 + hi)));
    f32x16 s_cur;
    {
        f16x8 kf[8];
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) kf[dk] = k_frag(lds, dk);
#pragma unroll
        for (int r = 0; r < 16; ++r) s_cur[r] = 0.0f;
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) s_cur = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[dk], qf[dk], s_cur, 0, 0, 0);
    }
    if (diag(0)) mask_tile(s_cur, q_lim, (int)(kh * 32 - qfirst), hi);

    // Iteration kb: block kb+1 has landed (barrier), block kb+3 is requested into the stage
    // of block kb-1 (read by every wave before the barrier), then the QK MFMAs of block
    // kb+1 run interleaved with the exponentials of block kb, and the PV MFMAs of block kb
    // with the sums. One barrier per iteration. Blocks past a wave's diagonal are computed
    // fully masked (p = 0) rather than skipped. Steady iterations (blocks kb+1..kb+3 exist,
    // block kb+1 lies wholly below this wave's diagonal) run a copy without those checks.
    // Unrolled by two so the score tiles swap roles by name.
    auto iteration = [&](int kb, auto steady_t, f32x16& s_cur, f32x16& s_nxt) {
        constexpr bool STEADY = decltype(steady_t)::value;
        // every LDS read of the previous iteration has completed (its stage is refilled below)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        if (STEADY || kb + 2 < nkb) wait_vm<4>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (STEADY || kb + 3 < nkb)
            issue_block(lds_a + ((kb + 3) & (NSTAGE - 1)) * STAGE, src, kp, vp, S, kb + 3, wave, lane);
        // Scores are in log2 units (q carries log2(e)/sqrt(128)). Lazy rescaling: the exponent
        // base m_run moves only when some query's block maximum exceeds it by more than TAU, so
        // every probability is at most 2^TAU (exact in fp16, no overflow in the fp32 sums) and
        // the rescale of l and the 64 accumulators runs only on the few blocks that raise a
        // base. The base cancels in the final division. -inf + TAU is -inf, so a query's first
        // visible key always sets its base.
        float mblk = s_cur[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mblk = fmaxf(mblk, s_cur[r]);
        mblk = max_halves(mblk);
        if (__builtin_amdgcn_ballot_w64(mblk > m_run + TAU)) {
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
        // QK MFMAs of block kb+1 (K fragments read 4 ahead) with the exponentials of block kb;
        // on the last block they run on a stale stage and their result is not used
        const unsigned char* st_n = stage_of(kb + 1);
        const unsigned char* st_c = stage_of(kb);
        f16x8 kf[8];
#pragma unroll
        for (int dk = 0; dk < 4; ++dk) kf[dk] = k_frag(st_n, dk);
        s_nxt = f32x16{};
        f16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(s_cur[r] - m_use);
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) {
            if (dk + 4 < 8) kf[dk + 4] = k_frag(st_n, dk + 4);
            s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[dk], qf[dk], s_nxt, 0, 0, 0);
        }
        // PV MFMAs of block kb (V fragments read 4 ahead)
        f16x8 vf[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) vf[j] = v_frag(st_c, j >> 2, j & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j + 4 < 8) vf[j + 4] = v_frag(st_c, (j + 4) >> 2, (j + 4) & 3);
            o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[j], pb[j >> 2], o[j & 3], 0, 0, 0);
        }
        // row sum of the fp16 probabilities that the PV MFMAs used (v_dot2_f32_f16 by ones)
        float lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const f16x2 pair = {pb[e >> 2][2 * (e & 3)], pb[e >> 2][2 * (e & 3) + 1]};
            lsum = __builtin_amdgcn_fdot2(pair, ones2, lsum, false);
        }
        l_run += sum_halves(lsum);
        if (!STEADY && kb + 1 < nkb && diag(kb + 1))
            mask_tile(s_nxt, q_lim, (int)((int64_t)(kb + 1) * KB + kh * 32 - qfirst), hi);
    };
    int steady_end = 0;
    while (steady_end + 3 < nkb && !diag(steady_end + 1)) ++steady_end;
    f32x16 s_nxt;
    for (int kb = 0; kb < nkb; kb += 2) {
        if (kb + 1 < steady_end) {
            iteration(kb, std::true_type{}, s_cur, s_nxt);
            iteration(kb + 1, std::true_type{}, s_nxt, s_cur);
        } else {
            iteration(kb, std::false_type{}, s_cur, s_nxt);
            if (kb + 1 < nkb) iteration(kb + 1, std::false_type{}, s_nxt, s_cur);
        }
    }
    __syncthreads();   // every wave is done with the stages; they now hold the exchange
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
