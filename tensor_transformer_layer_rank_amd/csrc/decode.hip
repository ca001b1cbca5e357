// Decode-step (one new token per sequence, M <= 64 rows) kernels of a rank's shard.
// The work is bound by streaming the weight shards and the KV cache from HBM once.
//
//   skinny_kernel        split-K GEMM A[M, K] . W[K, N] for small M. A workgroup owns a
//                        128-column strip and one K chunk; its 4 waves take interleaved 32-row
//                        steps, each streaming a 32 x 128 weight block with 128-bit loads
//                        (every weight byte read once, the next step's block already in
//                        flight), transposing it in registers (v_perm) and feeding
//                        v_mfma_f32_16x16x32_bf16 with the activations as the A operand. The
//                        waves' partials meet in LDS; each wave then sums a quarter of the rows
//                        in wave order and writes it to the chunk's fp32 partial buffer.
//   reduce kernels       sum the chunk partials in chunk order and apply the layer's
//                        epilogue: fp32/bf16 store (O and down partials, vocabulary-split
//                        logits) or SiLU(gate)*up.
//   decode_attn_kernel   the QKV partials' reduction (rotary embedding at the cache position,
//                        key and value appended to the cache) fused with the attention of
//                        the new token over cache slots 0..pos in a single pass: 16-lane
//                        groups stream 256-byte key and value rows with an online softmax
//                        each, merged in LDS at the end.
//
// Partial sums across workgroups go through HBM-resident buffers and a separate kernel:
// a device-scope fence per workgroup (L2 write-back and invalidate on this GPU) costs far
// more than the extra launch.
//
// Sources: the column/row split of "CUDA tensor parallel computations" (第二类, 第三类), the
// attention shard of its section 放进 Transformer, the per-rank KV cache of "TensorRT LLM
// 中的并行策略" (注意力模块), and the vocabulary-split output layer of "张量并行：切分
// Transformer 层的分布式训练" (输入与输出层).
#include <cmath>

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

// Grid of one launch: K is split so that the launch has ~256 workgroups (one per compute
// unit). Measured on the decode step: with the step's sub-layers as parallel graph branches,
// grids that leave each compute unit a second workgroup slot overlap better with the other
// branches than grids of ~512 workgroups, although the latter stream a lone GEMM faster.
SkinnyPlan plan_skinny(int64_t N, int64_t K, int nb) {
    SkinnyPlan p;
    p.strips_per_b = (N + STRIP - 1) / STRIP;
    p.strips = p.strips_per_b * nb;
    p.ncols = p.strips * STRIP;
    int64_t target = (256 + p.strips - 1) / p.strips;
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

struct SkinnyArgs {
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B1;
    const uint16_t* B2;      // second weight of the dual (gate/up) form
    int64_t M, N, K, kchunk, strips_per_b, ncols;
    int splits;
    float* part;             // [splits][M][ncols]
};

template <int MB>
struct StepRegs {
    u32x4 w[8];
    u32x4 a[MB];
    bool k_ok;   // this lane's 8 k rows lie inside the chunk (else its activations count as 0)
};

// Loads of one 32-row step: `wp` points at this lane's 8-column group in weight row kr
// (kr = k0 + 8 * grp), `ap` at this lane's activation rows, column kr. Every load is issued
// unconditionally, from an always-valid stand-in address (wsafe / asafe) where the element
// lies outside the matrix, and no loaded value is touched here: branch-free loads whose
// results are first used by the step's MFMAs let the compiler count outstanding loads
// exactly, so a step waits only for its own loads while the next step's are in flight.
// Outside elements cannot leak into stored results: columns past N and tokens past M only
// feed accumulators that are never stored, and rows past the chunk are cancelled by zeroing
// the activations (k_ok) when the MFMAs consume them. K chunks and K are multiples of 8, so
// a lane's 8 rows are all inside or all outside.
template <int MB>
__device__ __forceinline__ void load_step(StepRegs<MB>& s, const uint16_t* wp, const uint16_t* ap,
                                          const uint16_t* wsafe, const uint16_t* asafe,
                                          int64_t ldw, int64_t lda, int64_t kr, int64_t kend,
                                          bool col_ok, uint32_t m_ok) {
    s.k_ok = kr < kend;
    const bool w_ok = s.k_ok && col_ok;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        s.w[i] = *reinterpret_cast<const u32x4*>(w_ok ? wp + i * ldw : wsafe);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const bool ok = ((m_ok >> mb) & 1u) && s.k_ok;
        s.a[mb] = *reinterpret_cast<const u32x4*>(ok ? ap + mb * 16 * lda : asafe);
    }
}

// acc[mb][t][r] += A[m = mb*16 + 4*grp + r][kr..] . W[kr..][col + t]: the 8 x 8 block of
// weights a lane loaded (rows kr..kr+7, columns col..col+7) is transposed so that column t
// becomes the 8-k operand of MFMA t.
template <int MB>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[MB][8], const StepRegs<MB>& s) {
    bf16x8 a[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        a[mb] = __builtin_bit_cast(bf16x8, s.k_ok ? s.a[mb] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const unsigned sel = (t & 1) ? 0x07060302u : 0x05040100u;
        u32x4 bt;
        bt.x = __builtin_amdgcn_perm(s.w[1][t >> 1], s.w[0][t >> 1], sel);
        bt.y = __builtin_amdgcn_perm(s.w[3][t >> 1], s.w[2][t >> 1], sel);
        bt.z = __builtin_amdgcn_perm(s.w[5][t >> 1], s.w[4][t >> 1], sel);
        bt.w = __builtin_amdgcn_perm(s.w[7][t >> 1], s.w[6][t >> 1], sel);
        const bf16x8 b = __builtin_bit_cast(bf16x8, bt);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            acc[mb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[mb][t], 0, 0, 0);
    }
}

template <int MB>
__global__ __launch_bounds__(256, MB <= 2 ? 2 : 1) void skinny_kernel(SkinnyArgs g) {
    __shared__ f32x4 red[4][MB * 16][STRIP / 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const int64_t strip = blockIdx.x, split = blockIdx.y;
    const bool second = strip >= g.strips_per_b;
    const uint16_t* Bp = second ? g.B2 : g.B1;
    const int64_t cgroup = strip % g.strips_per_b;
    const int64_t c0 = cgroup * STRIP;
    const int64_t col = c0 + 8 * l16;
    const bool col_ok = col < g.N;
    const int64_t kbeg = split * g.kchunk;
    const int64_t kend = (kbeg + g.kchunk < g.K) ? kbeg + g.kchunk : g.K;

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // waves take steps wave, wave+4, ...; two register sets keep the next step in flight
    uint32_t m_ok = 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) m_ok |= (mb * 16 + l16 < g.M) ? (1u << mb) : 0u;
    const int64_t kfirst = kbeg + wave * STEP + 8 * grp;
    const uint16_t* wp = Bp + kfirst * g.N + col;          // advances 4 steps at a time
    const uint16_t* ap = g.A + (int64_t)l16 * g.lda + kfirst;
    const int64_t wstep = 4 * STEP * g.N, astep = 4 * STEP;
    // in-bounds stand-ins: row kbeg of this lane's column group (or of the strip's first
    // group), and token row 0 at column kbeg
    const uint16_t* wsafe = Bp + kbeg * g.N + (col_ok ? col : c0);
    const uint16_t* asafe = g.A + kbeg;
    StepRegs<MB> s0, s1;
    int64_t kr = kfirst;
    if (kr - 8 * grp < kend) load_step<MB>(s0, wp, ap, wsafe, asafe, g.N, g.lda, kr, kend, col_ok, m_ok);
    for (; kr - 8 * grp < kend; kr += 8 * STEP) {
        // the next two steps are loaded whether or not they exist (see load_step); the
        // scheduling barriers keep each step's loads issued before the previous step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
        load_step<MB>(s1, wp + wstep, ap + astep, wsafe, asafe, g.N, g.lda, kr + 4 * STEP, kend, col_ok, m_ok);
        __builtin_amdgcn_sched_barrier(0);
        mma_step<MB>(acc, s0);
        __builtin_amdgcn_sched_barrier(0);
        load_step<MB>(s0, wp + 2 * wstep, ap + 2 * astep, wsafe, asafe, g.N, g.lda, kr + 8 * STEP, kend, col_ok,
                      m_ok);
        __builtin_amdgcn_sched_barrier(0);
        if (kr + 4 * STEP - 8 * grp < kend) mma_step<MB>(acc, s1);
        wp += 2 * wstep;
        ap += 2 * astep;
    }

    // every wave's partial goes to LDS; after one barrier each wave sums a quarter of the rows
    // over the four waves' partials in wave order and stores it (all waves store at once)
    // acc[mb][t][r] = C[m = mb*16 + 4*grp + r][c0 + 8*l16 + t]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + 4 * grp + r;
            red[wave][m][2 * l16] = f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            red[wave][m][2 * l16 + 1] = f32x4{acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
        }
    __syncthreads();
    constexpr int ROWS = MB * 16 / 4;   // rows per wave
    float* dst = g.part + (split * g.M) * g.ncols + strip * STRIP;
#pragma unroll
    for (int rr = lane >> 3; rr < ROWS; rr += 8) {   // lane: row rr, 16-byte chunks lane%8 + 8q
        const int m = wave * ROWS + rr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = (lane & 7) + 8 * q;
            f32x4 v = red[0][m][c];
            v += red[1][m][c];
            v += red[2][m][c];
            v += red[3][m][c];
            if (m < g.M) *reinterpret_cast<f32x4*>(dst + m * g.ncols + 4 * c) = v;
        }
    }
}

// v[i] = sum over chunks (in order) of part[s][m][c[i]] for NC columns of row m. The chunks'
// values are loaded 8 at a time for all NC columns together, unconditionally (chunk indexes
// past the last one re-read the last), so that a thread waits for one memory round trip per
// 8 chunks rather than one per chunk and column.
template <int NC>
__device__ __forceinline__ void sum_splits(const float* part, int splits, int64_t M, int64_t ncols,
                                           int64_t m, const int64_t (&c)[NC], float (&v)[NC]) {
    constexpr int U = 8;
    const float* p = part + m * ncols;
    const int64_t stride = M * ncols;
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += U) {
        float t[U][NC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float* ps = p + (int64_t)(s0 + u < splits ? s0 + u : splits - 1) * stride;
#pragma unroll
            for (int i = 0; i < NC; ++i) t[u][i] = ps[c[i]];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < NC; ++i)
                if (s0 + u < splits) v[i] = (s0 + u == 0) ? t[u][i] : v[i] + t[u][i];
    }
}

// kind: 0 fp32 store, 1 fp32 +=, 2 bf16, 3 bf16 ReLU
__global__ __launch_bounds__(256) void reduce_store_kernel(const float* __restrict__ part, int splits,
                                                           int64_t M, int64_t N, int64_t ncols, void* C,
                                                           int64_t ldc, int kind) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx - m * N;
    const int64_t cols[1] = {n};
    float sum[1];
    sum_splits<1>(part, splits, M, ncols, m, cols, sum);
    const float v = sum[0];
    const int64_t off = m * ldc + n;
    if (kind == 0) static_cast<float*>(C)[off] = v;
    else if (kind == 1) static_cast<float*>(C)[off] += v;
    else if (kind == 2) static_cast<uint16_t*>(C)[off] = f32_to_bf16(v);
    else static_cast<uint16_t*>(C)[off] = f32_to_bf16(v > 0.f ? v : 0.f);
}

__global__ __launch_bounds__(256) void reduce_swiglu_kernel(const float* __restrict__ part, int splits,
                                                            int64_t M, int64_t I, int64_t ncols,
                                                            int64_t up_off, uint16_t* __restrict__ h) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * I) return;
    const int64_t m = idx / I, c = idx - m * I;
    const int64_t cols[2] = {c, up_off + c};
    float sum[2];
    sum_splits<2>(part, splits, M, ncols, m, cols, sum);
    const float gt = sum[0], up = sum[1];
    h[idx] = f32_to_bf16(gt / (1.0f + __expf(-gt)) * up);
}

// cos / sin of the 64 rotary angles pos * theta^(-2i/128) of one position (formed in fp64
// on the host and passed by value)
struct RopeRow {
    float c[64], s[64];
};

// Decode attention, one workgroup per (sequence, q head), fused with the end of the QKV
// projection. With its first cached keys and values already requested, the workgroup sums
// the split-K partials of its q head and of its kv head's new key and value (fixed chunk
// order, all loads of 8 chunks in flight together), rotates q and k by the angles of the cache
// position, and - if it is the first q head of its kv group - appends the new key and
// value (bf16) at that slot. It then attends in one pass: the 32 lane groups (16 lanes x 8
// dims = one 256-byte key or value row per group) stream cache slots grp, grp+32, ... four
// at a time (the next four in flight while the current ones are consumed), each group
// keeping its own online softmax (running max in log2 units, sum, 128-dim output); the new
// token's own key and value enter from LDS in fp32 (never read back from the cache, which
// another workgroup of the group may still be writing). The groups are merged in LDS and
// the normalised row is written as bf16.
// Sum over the 16 lanes of a row (lane group) with DPP moves folded into the adds: swap
// neighbours, swap pairs, mirror within 8, mirror within 16. Every lane ends with the same
// bits (each step adds the same two values, in either order).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    return v;
}

constexpr int DU = 4;     // keys per group per iteration
constexpr int NGRP = 32;  // 16-lane groups per workgroup

struct QkvPartials {
    const float* part;   // [splits][B][ncols]: columns [q heads | k heads | v heads] x 128
    int splits;
    int64_t ncols;
};

__global__ __launch_bounds__(NGRP * 16) void decode_attn_kernel(QkvPartials qp, RopeRow rope,
                                                                int hq, int hkv, int64_t pos,
                                                                int64_t cap, uint16_t* __restrict__ kc,
                                                                uint16_t* __restrict__ vc,
                                                                uint16_t* __restrict__ out) {
    __shared__ float red_o[NGRP][128];
    __shared__ float red_m[NGRP], red_l[NGRP];
    __shared__ float qs[128], kn[128], vn[128];
    const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t B = gridDim.y;
    const int g = (h * hkv) / hq;
    const uint16_t* kb = kc + ((b * hkv + g) * cap) * 128 + 8 * l16;
    const uint16_t* vb = vc + ((b * hkv + g) * cap) * 128 + 8 * l16;
    const int64_t L = pos;   // cached keys 0..pos-1
    // keys past L are read from row L-1 (branch-free) and masked when consumed
    auto load = [&](u32x4 (&kk)[DU], u32x4 (&vv)[DU], int64_t j0) {
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            const int64_t j = j0 + NGRP * u;
            const int64_t jj = j < L ? j : L - 1;
            kk[u] = *reinterpret_cast<const u32x4*>(kb + jj * 128);
            vv[u] = *reinterpret_cast<const u32x4*>(vb + jj * 128);
        }
    };
    // the group's first keys and values (slots < pos, which the append below never writes)
    // are requested before the QKV partials are summed, so the two round trips overlap
    u32x4 k0[DU], v0[DU];
    if (grp < L) load(k0, v0, grp);
    // q, new k (rotated pairs i, i+64) and new v of this head from the chunk partials
    if (tid < 64) {
        const int i = tid;
        const float c = rope.c[i], sn = rope.s[i];
        const int64_t cq = (int64_t)h * 128 + i, ck = (int64_t)(hq + g) * 128 + i;
        const int64_t cols[4] = {cq, cq + 64, ck, ck + 64};
        float x[4];
        sum_splits<4>(qp.part, qp.splits, B, qp.ncols, b, cols, x);
        qs[i] = x[0] * c - x[1] * sn;
        qs[i + 64] = x[1] * c + x[0] * sn;
        kn[i] = x[2] * c - x[3] * sn;
        kn[i + 64] = x[3] * c + x[2] * sn;
    } else if (tid < 128) {
        const int d = tid - 64;
        const int64_t cv = (int64_t)(hq + hkv + g) * 128 + d;
        const int64_t cols[2] = {cv, cv + 64};
        float x[2];
        sum_splits<2>(qp.part, qp.splits, B, qp.ncols, b, cols, x);
        vn[d] = x[0];
        vn[d + 64] = x[1];
    }
    __syncthreads();
    const int64_t slot = ((b * hkv + g) * cap + pos) * 128;
    if (h % (hq / hkv) == 0 && tid < 128) {
        kc[slot + tid] = f32_to_bf16(kn[tid]);
        vc[slot + tid] = f32_to_bf16(vn[tid]);
    }

    float m = -__builtin_inff(), l = 0.f, acc[8] = {};
    const float scale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qs[8 * l16 + e] * scale;
    // score of the new key (every group forms it; the 16 lanes of a group share it)
    float s_new = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s_new += qv[e] * kn[8 * l16 + e];
    s_new = sum16(s_new);

    auto consume = [&](const u32x4 (&kk)[DU], const u32x4 (&vv)[DU], int64_t j0) {
        float sc[DU];
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            float s = qv[0] * bf16_lo(kk[u].x) + qv[1] * bf16_hi(kk[u].x);
            s += qv[2] * bf16_lo(kk[u].y) + qv[3] * bf16_hi(kk[u].y);
            s += qv[4] * bf16_lo(kk[u].z) + qv[5] * bf16_hi(kk[u].z);
            s += qv[6] * bf16_lo(kk[u].w) + qv[7] * bf16_hi(kk[u].w);
            sc[u] = s;
        }
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            sc[u] = sum16(sc[u]);
            if (j0 + NGRP * u >= L) sc[u] = -__builtin_inff();
        }
        float mc = sc[0];
#pragma unroll
        for (int u = 1; u < DU; ++u) mc = fmaxf(mc, sc[u]);
        const float m_new = fmaxf(m, mc);                    // finite: key j0 < L is real
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        float p[DU], ps = 0.f;
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            p[u] = __builtin_amdgcn_exp2f(sc[u] - m_new);
            ps += p[u];
        }
        l = l * alpha + ps;
        m = m_new;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
        for (int u = 0; u < DU; ++u) {
            acc[0] += p[u] * bf16_lo(vv[u].x);
            acc[1] += p[u] * bf16_hi(vv[u].x);
            acc[2] += p[u] * bf16_lo(vv[u].y);
            acc[3] += p[u] * bf16_hi(vv[u].y);
            acc[4] += p[u] * bf16_lo(vv[u].z);
            acc[5] += p[u] * bf16_hi(vv[u].z);
            acc[6] += p[u] * bf16_lo(vv[u].w);
            acc[7] += p[u] * bf16_hi(vv[u].w);
        }
    };
    // two register sets: the next DU keys of the group are in flight while the current ones
    // are consumed
    u32x4 k1[DU], v1[DU];
    for (int64_t j0 = grp; j0 < L; j0 += 2 * NGRP * DU) {
        __builtin_amdgcn_sched_barrier(0);
        load(k1, v1, j0 + NGRP * DU);
        __builtin_amdgcn_sched_barrier(0);
        consume(k0, v0, j0);
        __builtin_amdgcn_sched_barrier(0);
        load(k0, v0, j0 + 2 * NGRP * DU);
        __builtin_amdgcn_sched_barrier(0);
        if (j0 + NGRP * DU < L) consume(k1, v1, j0 + NGRP * DU);
    }
    // merge the groups (a group without keys has m = -inf and weight 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[grp][8 * l16 + e] = acc[e];
    if (l16 == 0) {
        red_m[grp] = m;
        red_l[grp] = l;
    }
    __syncthreads();
    if (tid < 128) {
        float M = s_new;   // the new key: one more "group" with max s_new, sum 1, output v_new
        for (int r = 0; r < NGRP; ++r) M = fmaxf(M, red_m[r]);
        const float w_new = __builtin_amdgcn_exp2f(s_new - M);
        float num = w_new * vn[tid], den = w_new;
        for (int r = 0; r < NGRP; ++r) {
            const float w = __builtin_amdgcn_exp2f(red_m[r] - M);
            num += w * red_o[r][tid];
            den += w * red_l[r];
        }
        out[(b * hq + h) * 128 + tid] = f32_to_bf16(num / den);
    }
}

hipError_t skinny_run(SkinnyArgs& a, const SkinnyPlan& p, hipStream_t s, const char* name) {
    a.kchunk = p.kchunk;
    a.strips_per_b = p.strips_per_b;
    a.ncols = p.ncols;
    a.splits = (int)p.splits;
    dim3 grid((unsigned)p.strips, (unsigned)p.splits);
    ProfScope ps(name, s);
    if (a.M <= 32)
        skinny_kernel<2><<<grid, 256, 0, s>>>(a);
    else
        skinny_kernel<4><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
}

SkinnyArgs skinny_args(const void* A, const void* B1, const void* B2, float* part, int64_t M,
                       int64_t N, int64_t K, int64_t lda) {
    SkinnyArgs a{};
    a.A = static_cast<const uint16_t*>(A);
    a.lda = lda;
    a.B1 = static_cast<const uint16_t*>(B1);
    a.B2 = static_cast<const uint16_t*>(B2 ? B2 : B1);
    a.M = M;
    a.N = N;
    a.K = K;
    a.part = part;
    return a;
}

}  // namespace

size_t skinny_partials_bytes(int64_t M, int64_t N, int64_t K) {
    const SkinnyPlan p = plan_skinny(N, K, 1);
    return (size_t)(p.splits * M * p.ncols) * sizeof(float);
}
size_t skinny_swiglu_partials_bytes(int64_t M, int64_t I, int64_t H) {
    const SkinnyPlan p = plan_skinny(I, H, 2);
    return (size_t)(p.splits * M * p.ncols) * sizeof(float);
}

hipError_t skinny_linear(const void* A, const void* B, float* part, int64_t M, int64_t N, int64_t K,
                         int64_t lda, void* C, int64_t ldc, int kind, hipStream_t s) {
    SkinnyArgs a = skinny_args(A, B, nullptr, part, M, N, K, lda);
    const SkinnyPlan p = plan_skinny(N, K, 1);
    hipError_t e = skinny_run(a, p, s, "skinny_gemm");
    if (e != hipSuccess) return e;
    const int64_t n = M * N;
    ProfScope ps("skinny_reduce", s);
    reduce_store_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, (int)p.splits, M, N, p.ncols, C, ldc, kind);
    return hipGetLastError();
}

hipError_t skinny_swiglu(const void* X, const void* Wg, const void* Wu, float* part, void* h,
                         int64_t M, int64_t I, int64_t H, hipStream_t s) {
    SkinnyArgs a = skinny_args(X, Wg, Wu, part, M, I, H, H);
    const SkinnyPlan p = plan_skinny(I, H, 2);
    hipError_t e = skinny_run(a, p, s, "skinny_gemm_gateup");
    if (e != hipSuccess) return e;
    const int64_t n = M * I;
    ProfScope ps("skinny_reduce_swiglu", s);
    reduce_swiglu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, (int)p.splits, M, I, p.ncols,
                                                                     p.ncols / 2, static_cast<uint16_t*>(h));
    return hipGetLastError();
}

hipError_t decode_attn_step(const void* X, const void* Wqkv, float* part, int64_t B, int64_t H, int hq,
                            int hkv, int64_t pos, float theta, void* k_cache, void* v_cache, int64_t cap,
                            void* out, hipStream_t s) {
    const int64_t N = (int64_t)(hq + 2 * hkv) * 128;
    SkinnyArgs a = skinny_args(X, Wqkv, nullptr, part, B, N, H, H);
    const SkinnyPlan p = plan_skinny(N, H, 1);
    hipError_t e = skinny_run(a, p, s, "skinny_gemm_qkv");
    if (e != hipSuccess) return e;
    RopeRow rope;
    for (int i = 0; i < 64; ++i) {
        const double ang = (double)pos * std::pow((double)theta, -2.0 * (double)i / 128.0);
        rope.c[i] = (float)std::cos(ang);
        rope.s[i] = (float)std::sin(ang);
    }
    const QkvPartials qp{part, (int)p.splits, p.ncols};
    ProfScope ps("decode_attn", s);
    decode_attn_kernel<<<dim3((unsigned)hq, (unsigned)B), NGRP * 16, 0, s>>>(
        qp, rope, hq, hkv, pos, cap, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
        static_cast<uint16_t*>(out));
    return hipGetLastError();
}

}  // namespace tpk
