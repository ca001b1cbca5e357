// Decode-step (one new token per sequence, M <= 64 rows) kernels of a rank's shard.
// The work is bound by streaming the weight shards and the KV cache from HBM once.
//
//   skinny_kernel        split-K GEMM A[M, K] . W[K, N] for small M. A workgroup owns a
//                        128-column strip and one K chunk; its 4 waves take 32-row steps, each
//                        streaming a 32 x 128 weight block with 128-bit loads (every weight byte
//                        read once, the next step's block already in flight), transposing it in
//                        registers (v_perm) and feeding v_mfma_f32_16x16x32_bf16 with the
//                        activations as the A operand. For M <= 32 the waves take interleaved
//                        128-row groups and stage the activation rows through LDS (whole 256-byte
//                        rows per load); for larger M they interleave 32-row steps and load the
//                        fragments directly. The waves' partials meet in LDS;
//                        each wave then sums a quarter of the rows in wave order and writes it to
//                        the chunk's fp32 partial buffer.
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
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
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

// Weight and cache rows are read once per step, so they are loaded nontemporal (streamed past
// the caches): the activation rows that every workgroup re-reads stay cached. Measured on the
// 7B decode step: attention 52 -> 49 us, the GEMM launches 1-3% faster.
__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

struct SkinnyArgs {
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B1;
    const uint16_t* B2;      // second weight of the dual (gate/up) form
    int64_t M, N, K, kchunk, strips_per_b, ncols;
    int splits;
    int strips;              // strips per K chunk (dual: gate strips then up strips)
    int wg0;                 // first workgroup of this GEMM in a launch over several
    float* part;             // [splits][strips][M][128]: one contiguous block per workgroup
    int packed;              // weights in 128-column strips: [strip][K][128] (else [K][N])
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
        s.w[i] = ld_stream(w_ok ? wp + i * ldw : wsafe);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const bool ok = ((m_ok >> mb) & 1u) && s.k_ok;
        s.a[mb] = *reinterpret_cast<const u32x4*>(ok ? ap + mb * 16 * lda : asafe);
    }
}

// acc[mb][t][r] += A[m = mb*16 + 4*grp + r][kr..] . W[kr..][col + t]: the 8 x 8 block of
// weights a lane loaded (rows kr..kr+7, columns col..col+7) is transposed so that column t
// becomes the 8-k operand of MFMA t. F16: the 16-bit operands are IEEE half values.
template <int MB, bool F16>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[MB][8], const StepRegs<MB>& s) {
    u32x4 a[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = s.k_ok ? s.a[mb] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const unsigned sel = (t & 1) ? 0x07060302u : 0x05040100u;
        u32x4 bt;
        bt.x = __builtin_amdgcn_perm(s.w[1][t >> 1], s.w[0][t >> 1], sel);
        bt.y = __builtin_amdgcn_perm(s.w[3][t >> 1], s.w[2][t >> 1], sel);
        bt.z = __builtin_amdgcn_perm(s.w[5][t >> 1], s.w[4][t >> 1], sel);
        bt.w = __builtin_amdgcn_perm(s.w[7][t >> 1], s.w[6][t >> 1], sel);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if constexpr (F16)
                acc[mb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[mb]),
                                                                    __builtin_bit_cast(f16x8, bt), acc[mb][t], 0, 0, 0);
            else
                acc[mb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb]),
                                                                     __builtin_bit_cast(bf16x8, bt), acc[mb][t], 0, 0, 0);
        }
    }
}

// One workgroup's strip and K chunk of GEMM g.
template <int MB, bool F16>
__device__ __forceinline__ void skinny_body(const SkinnyArgs& g, int64_t strip, int64_t split,
                                            f32x4 (&red)[4][MB * 16][STRIP / 4]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
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
    // weight rows: [K][N] in place, or the strip's own [K][128] block when packed
    const int64_t ldw = g.packed ? STRIP : g.N;
    const uint16_t* Bs = g.packed ? Bp + cgroup * g.K * STRIP : Bp;
    const int64_t colw = g.packed ? 8 * l16 : col;
    const uint16_t* wp = Bs + kfirst * ldw + colw;         // advances 4 steps at a time
    const uint16_t* ap = g.A + (int64_t)l16 * g.lda + kfirst;
    const int64_t wstep = 4 * STEP * ldw, astep = 4 * STEP;
    // in-bounds stand-ins: row kbeg of this lane's column group (or of the strip's first
    // group), and token row 0 at column kbeg
    const uint16_t* wsafe = Bs + kbeg * ldw + (col_ok ? colw : colw - 8 * l16);
    const uint16_t* asafe = g.A + kbeg;
    StepRegs<MB> s0, s1;
    int64_t kr = kfirst;
    if (kr - 8 * grp < kend) load_step<MB>(s0, wp, ap, wsafe, asafe, ldw, g.lda, kr, kend, col_ok, m_ok);
    for (; kr - 8 * grp < kend; kr += 8 * STEP) {
        // the next two steps are loaded whether or not they exist (see load_step); the
        // scheduling barriers keep each step's loads issued before the previous step's MFMAs
        __builtin_amdgcn_sched_barrier(0);
        load_step<MB>(s1, wp + wstep, ap + astep, wsafe, asafe, ldw, g.lda, kr + 4 * STEP, kend, col_ok, m_ok);
        __builtin_amdgcn_sched_barrier(0);
        mma_step<MB, F16>(acc, s0);
        __builtin_amdgcn_sched_barrier(0);
        load_step<MB>(s0, wp + 2 * wstep, ap + 2 * astep, wsafe, asafe, ldw, g.lda, kr + 8 * STEP, kend, col_ok,
                      m_ok);
        __builtin_amdgcn_sched_barrier(0);
        if (kr + 4 * STEP - 8 * grp < kend) mma_step<MB, F16>(acc, s1);
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
    float* dst = g.part + (split * g.M) * g.ncols + strip * g.M * STRIP;
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
            if (m < g.M) *reinterpret_cast<f32x4*>(dst + m * STRIP + 4 * c) = v;
        }
    }
}

// The same for M <= 32 (MB = 2), with the activations staged through LDS: wave w takes the
// 128-row groups w, w + 4, ... of the chunk (4 steps each; 128-row interleaving keeps the four
// waves on neighbouring weight rows, which streamed faster than contiguous quarters). For each
// group it loads the activation block A[0..31][128 k] with whole 256-byte rows (16 lanes per
// row, 4 rows per instruction: 1 KB of contiguous bytes each, instead of 16 rows x 64 bytes per
// MFMA fragment load), writes it to its own LDS region (16-byte chunk c of row r at chunk
// position c ^ (r & 15)) and reads the MFMA fragments from there. The next group's block is in
// flight in registers meanwhile. No barrier: each wave reads only what it wrote. Measured on the
// 7B decode step: 0.131 -> 0.127 ms (the fragment loads' scattered cache lines cost ~8 us in all;
// whole-row loads recover part of it).
template <bool F16>
__device__ __forceinline__ void skinny_body_lds(const SkinnyArgs& g, int64_t strip, int64_t split,
                                                f32x4 (&red)[4][32][STRIP / 4]) {
    constexpr int MB = 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const bool second = strip >= g.strips_per_b;
    const uint16_t* Bp = second ? g.B2 : g.B1;
    const int64_t cgroup = strip % g.strips_per_b;
    const int64_t c0 = cgroup * STRIP;
    const int64_t col = c0 + 8 * l16;
    const bool col_ok = col < g.N;
    const int64_t kbeg = split * g.kchunk;
    const int64_t kend = (kbeg + g.kchunk < g.K) ? kbeg + g.kchunk : g.K;
    // wave w takes 128-row groups w, w + 4, ... of the chunk
    const int64_t wbeg = kbeg + wave * 4 * STEP;
    const int64_t wend = kend;
    const int ngw = wend > wbeg ? (int)((wend - wbeg + 16 * STEP - 1) / (16 * STEP)) : 0;
    const int nst = 4 * ngw;

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    unsigned char* stg = reinterpret_cast<unsigned char*>(&red[wave][0][0]);   // 16 KB: two 8 KB blocks
    // weight rows: [K][N] in place, or the strip's own [K][128] block when packed
    const int64_t ldw = g.packed ? STRIP : g.N;
    const uint16_t* Bs = g.packed ? Bp + cgroup * g.K * STRIP : Bp;
    const int64_t colw = g.packed ? 8 * l16 : col;
    const uint16_t* wsafe = Bs + kbeg * ldw + (col_ok ? colw : colw - 8 * l16);
    const uint16_t* asafe = g.A + kbeg;
    // this lane's weight rows of step i (step i & 3 of group i >> 2): 8 grp .. + 7 of it
    auto load_w = [&](StepRegs<MB>& s, int i) {
        const int64_t kr = wbeg + (int64_t)(i >> 2) * 16 * STEP + (i & 3) * STEP + 8 * grp;
        s.k_ok = kr < wend;
        const bool ok = s.k_ok && col_ok;
        const uint16_t* wp = Bs + kr * ldw + colw;
#pragma unroll
        for (int r = 0; r < 8; ++r) s.w[r] = ld_stream(ok ? wp + r * ldw : wsafe);
    };
    // activation block of group G: row 4 j + (lane >> 4), 16-byte chunk lane & 15 of its 128 k
    u32x4 areg[8];
    auto load_a = [&](int G) {
        const int64_t k = wbeg + (int64_t)G * 16 * STEP + 8 * (lane & 15);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 4 * j + (lane >> 4);
            const bool ok = row < g.M && k < wend;
            areg[j] = *reinterpret_cast<const u32x4*>(ok ? g.A + (int64_t)row * g.lda + k : asafe);
        }
    };
    auto store_a = [&](int G) {
        unsigned char* base = stg + (G & 1) * 8192;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 4 * j + (lane >> 4);
            *reinterpret_cast<u32x4*>(base + row * 256 + (((lane & 15) ^ (row & 15)) << 4)) = areg[j];
        }
    };
    // fragments of step t (0..3) of group G: row l16 + 16 mb, k chunk 4 t + grp
    auto frag_a = [&](StepRegs<MB>& s, int G, int t) {
        const unsigned char* base = stg + (G & 1) * 8192;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = l16 + 16 * mb;
            s.a[mb] = *reinterpret_cast<const u32x4*>(base + row * 256 + (((4 * t + grp) ^ (row & 15)) << 4));
        }
    };
    StepRegs<MB> s0, s1;
    if (nst > 0) {
        load_a(0);
        load_w(s0, 0);
    }
    for (int G = 0; 4 * G < nst; ++G) {
        // every load below is issued whether or not its step exists (stand-in addresses, masked
        // by k_ok), so each wave's loop body is branch-free and the load counts stay exact
        __builtin_amdgcn_sched_barrier(0);
        store_a(G);
        load_a(G + 1);
        __builtin_amdgcn_sched_barrier(0);
        load_w(s1, 4 * G + 1);
        frag_a(s0, G, 0);
        mma_step<MB, F16>(acc, s0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(s0, 4 * G + 2);
        frag_a(s1, G, 1);
        mma_step<MB, F16>(acc, s1);
        __builtin_amdgcn_sched_barrier(0);
        load_w(s1, 4 * G + 3);
        frag_a(s0, G, 2);
        mma_step<MB, F16>(acc, s0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(s0, 4 * G + 4);
        frag_a(s1, G, 3);
        mma_step<MB, F16>(acc, s1);
    }

    // every wave's partial goes to LDS (its own staging region: the slot it owns in `red`)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + 4 * grp + r;
            red[wave][m][2 * l16] = f32x4{acc[mb][0][r], acc[mb][1][r], acc[mb][2][r], acc[mb][3][r]};
            red[wave][m][2 * l16 + 1] = f32x4{acc[mb][4][r], acc[mb][5][r], acc[mb][6][r], acc[mb][7][r]};
        }
    __syncthreads();
    constexpr int ROWS = MB * 16 / 4;
    float* dst = g.part + (split * g.M) * g.ncols + strip * g.M * STRIP;
#pragma unroll
    for (int rr = lane >> 3; rr < ROWS; rr += 8) {
        const int m = wave * ROWS + rr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = (lane & 7) + 8 * q;
            f32x4 v = red[0][m][c];
            v += red[1][m][c];
            v += red[2][m][c];
            v += red[3][m][c];
            if (m < g.M) *reinterpret_cast<f32x4*>(dst + m * STRIP + 4 * c) = v;
        }
    }
}

// Up to three GEMMs that share M in one launch (a one-dimensional grid): workgroups g1.wg0..
// belong to g1, g2.wg0.. to g2, the rest to g0; within a GEMM, workgroup w takes strip
// w % strips of K chunk w / strips. The GEMM is picked by scalar selects over the three
// argument slots (the argument block is never indexed dynamically).
template <int MB, bool F16>
__global__ __launch_bounds__(256, MB <= 2 ? 2 : 1) void skinny_kernel(SkinnyArgs g0, SkinnyArgs g1, SkinnyArgs g2,
                                                                     int n) {
    __shared__ f32x4 red[4][MB * 16][STRIP / 4];
    const int bid = (int)blockIdx.x;
    const bool s2 = n > 2 && bid >= g2.wg0, s1 = !s2 && n > 1 && bid >= g1.wg0;
    SkinnyArgs g;
#define TP_SEL(f) g.f = s2 ? g2.f : (s1 ? g1.f : g0.f)
    TP_SEL(A);
    TP_SEL(lda);
    TP_SEL(B1);
    TP_SEL(B2);
    TP_SEL(M);
    TP_SEL(N);
    TP_SEL(K);
    TP_SEL(kchunk);
    TP_SEL(strips_per_b);
    TP_SEL(ncols);
    TP_SEL(splits);
    TP_SEL(strips);
    TP_SEL(wg0);
    TP_SEL(part);
    TP_SEL(packed);
#undef TP_SEL
    const int local = bid - g.wg0;
    if constexpr (MB == 2)
        skinny_body_lds<F16>(g, local % g.strips, local / g.strips, red);
    else
        skinny_body<MB, F16>(g, local % g.strips, local / g.strips, red);
}

// v[i] = sum over chunks (in order) of part[s][m][c[i]] for NC columns of row m. The chunks'
// values are loaded 8 at a time for all NC columns together, unconditionally (chunk indexes
// past the last one re-read the last), so that a thread waits for one memory round trip per
// 8 chunks rather than one per chunk and column.
// offset of element (row m, column c) inside one chunk's partials [strips][M][128]
__device__ __forceinline__ int64_t part_ofs(int64_t m, int64_t c, int64_t M) {
    return (c >> 7) * M * STRIP + m * STRIP + (c & (STRIP - 1));
}

template <int NC>
__device__ __forceinline__ void sum_splits(const float* part, int splits, int64_t M, int64_t ncols,
                                           int64_t m, const int64_t (&c)[NC], float (&v)[NC]) {
    constexpr int U = 8;
    const int64_t stride = M * ncols;
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += U) {
        float t[U][NC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float* ps = part + (int64_t)(s0 + u < splits ? s0 + u : splits - 1) * stride;
#pragma unroll
            for (int i = 0; i < NC; ++i) t[u][i] = ps[part_ofs(m, c[i], M)];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < NC; ++i)
                if (s0 + u < splits) v[i] = (s0 + u == 0) ? t[u][i] : v[i] + t[u][i];
    }
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// kind: 0 fp32 store, 1 fp32 +=, 2 bf16, 3 bf16 ReLU, 5 fp16, 6 fp16 ReLU, 7 fp32 ReLU
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
    else if (kind == 3) static_cast<uint16_t*>(C)[off] = f32_to_bf16(v > 0.f ? v : 0.f);
    else if (kind == 5) static_cast<uint16_t*>(C)[off] = f32_to_f16(v);
    else if (kind == 6) static_cast<uint16_t*>(C)[off] = f32_to_f16(v > 0.f ? v : 0.f);
    else static_cast<float*>(C)[off] = v > 0.f ? v : 0.f;
}

__global__ __launch_bounds__(256) void reduce_swiglu_kernel(const float* __restrict__ part, int splits,
                                                            int64_t M, int64_t I, int64_t ncols,
                                                            int64_t up_off, uint16_t* __restrict__ h, int h16) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * I) return;
    const int64_t m = idx / I, c = idx - m * I;
    const int64_t cols[2] = {c, up_off + c};
    float sum[2];
    sum_splits<2>(part, splits, M, ncols, m, cols, sum);
    const float gt = sum[0], up = sum[1];
    const float v = gt / (1.0f + __expf(-gt)) * up;
    h[idx] = h16 ? f32_to_f16(v) : f32_to_bf16(v);
}

// One output of a reduce launch over several: the chunk partials of a skinny GEMM summed in
// chunk order, then kind 0 fp32 store, 1 fp32 +=, 2 bf16, 3 bf16 ReLU, 4 bf16 SiLU(gate) * up
// (gate column c and up column up_off + c of the partials; N = I).
struct ReduceOut {
    const float* part;
    int splits;
    int kind;
    int64_t N, ncols, up_off, ldc;
    void* C;
    int64_t e0;   // first element of this output in the launch
};

// element e of one output: the chunk partials summed in order, then the output's epilogue
__device__ __forceinline__ void reduce_one(const ReduceOut& r, int64_t M, int64_t e) {
    const int64_t m = e / r.N, c = e - m * r.N;
    const int64_t off = m * r.ldc + c;
    if (r.kind == 4) {
        const int64_t cols[2] = {c, r.up_off + c};
        float sum[2];
        sum_splits<2>(r.part, r.splits, M, r.ncols, m, cols, sum);
        const float gt = sum[0], up = sum[1];
        static_cast<uint16_t*>(r.C)[off] = f32_to_bf16(gt / (1.0f + __expf(-gt)) * up);
        return;
    }
    const int64_t cols[1] = {c};
    float sum[1];
    sum_splits<1>(r.part, r.splits, M, r.ncols, m, cols, sum);
    const float v = sum[0];
    if (r.kind == 0) static_cast<float*>(r.C)[off] = v;
    else if (r.kind == 1) static_cast<float*>(r.C)[off] += v;
    else if (r.kind == 2) static_cast<uint16_t*>(r.C)[off] = f32_to_bf16(v);
    else static_cast<uint16_t*>(r.C)[off] = f32_to_bf16(v > 0.f ? v : 0.f);
}

// Four consecutive fp32 outputs (kind 0 only): element e4 .. e4+3 of the launch, e4 % 4 == 0, every
// output's N and first element multiples of 4, partial rows and outputs 16-byte aligned. The sums
// are those of reduce_element, element by element (the same chunk order).
__global__ __launch_bounds__(256) void reduce4_store_kernel(ReduceOut r0, ReduceOut r1, ReduceOut r2, int n,
                                                            int64_t M, int64_t total) {
    const int64_t e4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e4 >= total) return;
    const bool s2 = n > 2 && e4 >= r2.e0, s1 = !s2 && n > 1 && e4 >= r1.e0;
    const float* part = s2 ? r2.part : (s1 ? r1.part : r0.part);
    const int splits = s2 ? r2.splits : (s1 ? r1.splits : r0.splits);
    const int64_t N = s2 ? r2.N : (s1 ? r1.N : r0.N);
    const int64_t ncols = s2 ? r2.ncols : (s1 ? r1.ncols : r0.ncols);
    const int64_t ldc = s2 ? r2.ldc : (s1 ? r1.ldc : r0.ldc);
    float* C = static_cast<float*>(s2 ? r2.C : (s1 ? r1.C : r0.C));
    const int64_t e = e4 - (s2 ? r2.e0 : (s1 ? r1.e0 : r0.e0));
    const int64_t m = e / N, c = e - m * N;
    constexpr int U = 8;
    const float* p = part + part_ofs(m, c, M);
    const int64_t stride = M * ncols;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += U) {
        f32x4 t[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            t[u] = *reinterpret_cast<const f32x4*>(p + (int64_t)(s0 + u < splits ? s0 + u : splits - 1) * stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s0 + u < splits) v = (s0 + u == 0) ? t[u] : v + t[u];
    }
    *reinterpret_cast<f32x4*>(C + m * ldc + c) = v;
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
    const float* part;   // [splits][strips][B][128]: columns [q heads | k heads | v heads] x 128
    int splits;
    int64_t ncols;
};

// Extra work a decode attention launch may carry: one more split-K reduction (output r, M rows,
// `total` elements; n = 0: none). Attention workgroup a takes elements a * per .. a * per + per - 1
// with its threads 128 and up, which have nothing else to do while threads 0..127 sum the QKV
// partials and the first cache rows are in flight, so the reduction needs no launch and no
// workgroups of its own.
constexpr int RED_THREADS = NGRP * 16 - 128;
struct AttnReduce {
    ReduceOut r;
    int n;
    int64_t M, total, per;
};

__global__ __launch_bounds__(NGRP * 16) void decode_attn_kernel(QkvPartials qp, RopeRow rope,
                                                                int hq, int hkv, int64_t B, int64_t pos,
                                                                int64_t cap, uint16_t* __restrict__ kc,
                                                                uint16_t* __restrict__ vc,
                                                                uint16_t* __restrict__ out, AttnReduce xr) {
    __shared__ float red_o[NGRP][128];
    __shared__ float red_m[NGRP], red_l[NGRP];
    __shared__ float qs[128], kn[128], vn[128];
    const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
    const int ab = (int)blockIdx.x;   // (sequence, q head)
    const int h = ab % hq;
    const int64_t b = ab / hq;
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
            kk[u] = ld_stream(kb + jj * 128);
            vv[u] = ld_stream(vb + jj * 128);
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
    } else if (xr.n) {
        const ReduceOut r = xr.r;   // a local copy: indexing through the argument block spills
        const int64_t e1 = (ab + 1) * xr.per < xr.total ? (ab + 1) * xr.per : xr.total;
        for (int64_t e = ab * xr.per + (tid - 128); e < e1; e += RED_THREADS) reduce_one(r, xr.M, e);
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

// Launch up to three prepared GEMMs (plan fields and wg0 filled in) as one grid of `wgs` workgroups.
hipError_t skinny_launch(const SkinnyArgs* a, int n, int wgs, int64_t M, hipStream_t s, const char* name, bool f16) {
    const SkinnyArgs g0 = a[0], g1 = n > 1 ? a[1] : a[0], g2 = n > 2 ? a[2] : a[0];
    ProfScope ps(name, s);
    if (f16) {
        if (M <= 32)
            skinny_kernel<2, true><<<(unsigned)wgs, 256, 0, s>>>(g0, g1, g2, n);
        else
            skinny_kernel<4, true><<<(unsigned)wgs, 256, 0, s>>>(g0, g1, g2, n);
    } else {
        if (M <= 32)
            skinny_kernel<2, false><<<(unsigned)wgs, 256, 0, s>>>(g0, g1, g2, n);
        else
            skinny_kernel<4, false><<<(unsigned)wgs, 256, 0, s>>>(g0, g1, g2, n);
    }
    return hipGetLastError();
}

// fill the plan fields of a (nb = 2 for the dual gate/up form) and place it at workgroup wg0
int skinny_place(SkinnyArgs& a, const SkinnyPlan& p, int wg0) {
    a.kchunk = p.kchunk;
    a.strips_per_b = p.strips_per_b;
    a.ncols = p.ncols;
    a.splits = (int)p.splits;
    a.strips = (int)p.strips;
    a.wg0 = wg0;
    return wg0 + (int)(p.strips * p.splits);
}

hipError_t skinny_run(SkinnyArgs& a, const SkinnyPlan& p, hipStream_t s, const char* name, bool f16 = false) {
    const int wgs = skinny_place(a, p, 0);
    return skinny_launch(&a, 1, wgs, a.M, s, name, f16);
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
                         int64_t lda, void* C, int64_t ldc, int kind, hipStream_t s, int f16_in) {
    SkinnyArgs a = skinny_args(A, B, nullptr, part, M, N, K, lda);
    const SkinnyPlan p = plan_skinny(N, K, 1);
    hipError_t e = skinny_run(a, p, s, "skinny_gemm", f16_in != 0);
    if (e != hipSuccess) return e;
    const int64_t n = M * N;
    ProfScope ps("skinny_reduce", s);
    reduce_store_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, (int)p.splits, M, N, p.ncols, C, ldc, kind);
    return hipGetLastError();
}

hipError_t skinny_swiglu(const void* X, const void* Wg, const void* Wu, float* part, void* h,
                         int64_t M, int64_t I, int64_t H, hipStream_t s, int f16) {
    SkinnyArgs a = skinny_args(X, Wg, Wu, part, M, I, H, H);
    const SkinnyPlan p = plan_skinny(I, H, 2);
    hipError_t e = skinny_run(a, p, s, "skinny_gemm_gateup", f16 != 0);
    if (e != hipSuccess) return e;
    const int64_t n = M * I;
    ProfScope ps("skinny_reduce_swiglu", s);
    reduce_swiglu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, (int)p.splits, M, I, p.ncols,
                                                                     p.ncols / 2, static_cast<uint16_t*>(h), f16);
    return hipGetLastError();
}

// W [K, N] (16-bit elements, row-major) -> P [ceil(N / 128)][K][128]: each 128-column strip of
// W as one contiguous block, columns past N zero. One thread copies 16 bytes.
__global__ __launch_bounds__(256) void pack_strips_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ P,
                                                          int64_t K, int64_t N, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 16-byte chunk of P
    if (i >= total) return;
    const int64_t j = i & 15, row = i >> 4;                              // row = strip * K + k
    const int64_t strip = row / K, k = row - strip * K;
    const int64_t col = strip * STRIP + 8 * j;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < N) v = *reinterpret_cast<const u32x4*>(W + k * N + col);
    *reinterpret_cast<u32x4*>(P + i * 8) = v;
}

size_t packed_strips_bytes(int64_t K, int64_t N) { return (size_t)((N + STRIP - 1) / STRIP) * K * STRIP * 2; }

hipError_t pack_strips(const void* W, int64_t K, int64_t N, void* P, hipStream_t s) {
    const int64_t total = (N + STRIP - 1) / STRIP * K * 16;
    ProfScope ps("pack_strips", s);
    pack_strips_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(static_cast<const uint16_t*>(W),
                                                                        static_cast<uint16_t*>(P), K, N, total);
    return hipGetLastError();
}

// ---- the whole decode step of a rank in four launches ------------------------------------
// K1: the projections that feed the attention and the MLP (QKV and gate/up) as one split-K launch;
// K2: decode attention (sums the QKV partials, RoPE, cache append, attention over the cache),
//     whose workgroups' spare threads meanwhile sum the gate/up partials through SiLU(gate) * up
//     into h;
// K3: O, down and the vocabulary-split head as one split-K launch (the head needs only X, but in
//     this launch its 2 * H * V bytes give the short O and down GEMMs company, so the launch's
//     start and end are spread over far more data);
// K4: the three sets of partials into Y_attn, Y_mlp and the logits.
namespace {

// Skinny launches are planned for two resident workgroups per compute unit (their reduction
// buffer takes 64 KB of LDS) on 256 compute units.
constexpr int64_t SLOTS = 512;
// Fixed cost of a round of workgroups (start, first round trip, LDS reduction, partial store) in
// units of weight rows of one strip
#ifndef TP_DECODE_ROUND_ROWS
#define TP_DECODE_ROUND_ROWS 256
#endif

// Common K chunk for the GEMMs of one launch (M activation rows): the multiple of 4 steps that
// minimises the estimated time, in weight rows of one strip streamed by one slot: a launch of w
// workgroups runs in ceil(w / SLOTS) rounds, each as long as a full chunk plus the fixed cost,
// and every workgroup's fp32 partials (M x 128, written once and read back once: as many bytes
// as 4M weight rows) share the bandwidth of all slots.
void plan_rounds(int64_t M, const int64_t* N, const int64_t* K, const int* nb, int n, SkinnyPlan* out) {
    int64_t best_kc = 4 * STEP, best_cost = -1;
    int64_t kmax = 0;
    for (int i = 0; i < n; ++i) kmax = K[i] > kmax ? K[i] : kmax;
    for (int64_t kc = 4 * STEP; kc < kmax + 4 * STEP; kc += 4 * STEP) {
        int64_t wgs = 0;
        for (int i = 0; i < n; ++i) wgs += (N[i] + STRIP - 1) / STRIP * nb[i] * ((K[i] + kc - 1) / kc);
        const int64_t cost =
            (wgs + SLOTS - 1) / SLOTS * (kc + TP_DECODE_ROUND_ROWS) + wgs * 4 * M / SLOTS;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_kc = kc;
        }
    }
    for (int i = 0; i < n; ++i) {
        SkinnyPlan& p = out[i];
        p.strips_per_b = (N[i] + STRIP - 1) / STRIP;
        p.strips = p.strips_per_b * nb[i];
        p.ncols = p.strips * STRIP;
        p.kchunk = best_kc;
        p.splits = (K[i] + best_kc - 1) / best_kc;
    }
}

struct DecodePlan {
    SkinnyPlan p1[2], p3[3];
    int n3;
    size_t off[7];   // qkv, gate/up partials, attention out, h, O, down, head partials
    size_t bytes;
};

DecodePlan plan_decode(int64_t B, int64_t H, int hq, int hkv, int64_t I, int64_t V) {
    DecodePlan d{};
    const int64_t nqkv = (int64_t)(hq + 2 * hkv) * 128, dq = (int64_t)hq * 128;
    const int64_t N1[2] = {nqkv, I}, K1[2] = {H, H};
    const int nb1[2] = {1, 2};
    plan_rounds(B, N1, K1, nb1, 2, d.p1);
    d.n3 = V > 0 ? 3 : 2;
    const int64_t N3[3] = {H, H, V}, K3[3] = {dq, I, H};
    const int nb3[3] = {1, 1, 1};
    plan_rounds(B, N3, K3, nb3, d.n3, d.p3);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t o = 0;
    auto take = [&](int i, size_t bytes) { d.off[i] = o; o += up(bytes); };
    take(0, (size_t)(d.p1[0].splits * B * d.p1[0].ncols) * 4);
    take(1, (size_t)(d.p1[1].splits * B * d.p1[1].ncols) * 4);
    take(2, (size_t)(B * dq) * 2);
    take(3, (size_t)(B * I) * 2);
    take(4, (size_t)(d.p3[0].splits * B * d.p3[0].ncols) * 4);
    take(5, (size_t)(d.p3[1].splits * B * d.p3[1].ncols) * 4);
    take(6, d.n3 > 2 ? (size_t)(d.p3[2].splits * B * d.p3[2].ncols) * 4 : 0);
    d.bytes = o;
    return d;
}

}  // namespace

size_t decode_step_ws_bytes(int64_t B, int64_t H, int hq, int hkv, int64_t I, int64_t V) {
    return plan_decode(B, H, hq, hkv, I, V).bytes;
}

hipError_t decode_step(const void* X, const void* Wqkv, const void* Wo, const void* Wg, const void* Wu,
                       const void* Wd, const void* Wlm, int64_t B, int64_t H, int hq, int hkv, int64_t I,
                       int64_t V, int64_t pos, float theta, void* k_cache, void* v_cache, int64_t cap, float* Ya,
                       float* Ym, float* logits, void* ws, hipStream_t s, bool packed) {
    const DecodePlan d = plan_decode(B, H, hq, hkv, I, V);
    unsigned char* base = static_cast<unsigned char*>(ws);
    float* part_qkv = reinterpret_cast<float*>(base + d.off[0]);
    float* part_gu = reinterpret_cast<float*>(base + d.off[1]);
    void* att = base + d.off[2];
    void* h = base + d.off[3];
    float* part_o = reinterpret_cast<float*>(base + d.off[4]);
    float* part_d = reinterpret_cast<float*>(base + d.off[5]);
    float* part_lm = reinterpret_cast<float*>(base + d.off[6]);
    const int64_t nqkv = (int64_t)(hq + 2 * hkv) * 128, dq = (int64_t)hq * 128;
    // K1
    SkinnyArgs a1[2] = {skinny_args(X, Wqkv, nullptr, part_qkv, B, nqkv, H, H),
                        skinny_args(X, Wg, Wu, part_gu, B, I, H, H)};
    int w = 0;
    for (int i = 0; i < 2; ++i) {
        w = skinny_place(a1[i], d.p1[i], w);
        a1[i].packed = packed;
    }
    hipError_t e = skinny_launch(a1, 2, w, B, s, "skinny_gemm_x", false);
    if (e != hipSuccess) return e;
    // K2: attention, with the gate/up reduction in the attention workgroups' spare threads
    RopeRow rope;
    for (int i = 0; i < 64; ++i) {
        const double ang = (double)pos * std::pow((double)theta, -2.0 * (double)i / 128.0);
        rope.c[i] = (float)std::cos(ang);
        rope.s[i] = (float)std::sin(ang);
    }
    {
        const QkvPartials qp{part_qkv, (int)d.p1[0].splits, d.p1[0].ncols};
        AttnReduce xr{};
        xr.r = ReduceOut{part_gu, (int)d.p1[1].splits, 4, I, d.p1[1].ncols, d.p1[1].ncols / 2, I, h, 0};
        xr.n = 1;
        xr.M = B;
        xr.total = B * I;
        xr.per = (xr.total + hq * B - 1) / (hq * B);
        ProfScope ps("decode_attn", s);
        decode_attn_kernel<<<(unsigned)(hq * B), NGRP * 16, 0, s>>>(
            qp, rope, hq, hkv, B, pos, cap, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
            static_cast<uint16_t*>(att), xr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // K3
    SkinnyArgs a3[3] = {skinny_args(att, Wo, nullptr, part_o, B, H, dq, dq),
                        skinny_args(h, Wd, nullptr, part_d, B, H, I, I),
                        skinny_args(X, Wlm, nullptr, part_lm, B, V, H, H)};
    w = 0;
    for (int i = 0; i < d.n3; ++i) {
        w = skinny_place(a3[i], d.p3[i], w);
        a3[i].packed = packed;
    }
    e = skinny_launch(a3, d.n3, w, B, s, "skinny_gemm_out", false);
    if (e != hipSuccess) return e;
    // K4
    const ReduceOut r0{part_o, (int)d.p3[0].splits, 0, H, d.p3[0].ncols, 0, H, Ya, 0};
    const ReduceOut r1{part_d, (int)d.p3[1].splits, 0, H, d.p3[1].ncols, 0, H, Ym, B * H};
    const ReduceOut r2{part_lm, d.n3 > 2 ? (int)d.p3[2].splits : 1, 0, V, d.n3 > 2 ? d.p3[2].ncols : 0, 0, V,
                       logits, 2 * B * H};
    const int64_t total = 2 * B * H + (d.n3 > 2 ? B * V : 0);
    ProfScope ps("skinny_reduce_out", s);
    reduce4_store_kernel<<<(unsigned)((total / 4 + 255) / 256), 256, 0, s>>>(r0, r1, r2, d.n3, B, total);
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
    decode_attn_kernel<<<(unsigned)(hq * B), NGRP * 16, 0, s>>>(
        qp, rope, hq, hkv, B, pos, cap, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
        static_cast<uint16_t*>(out), AttnReduce{});
    return hipGetLastError();
}

}  // namespace tpk
