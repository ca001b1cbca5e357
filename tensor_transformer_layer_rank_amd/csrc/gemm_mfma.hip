// MFMA GEMM tiles for gfx950, used by every prefill-size linear layer of a rank's shard,
// on bf16 operands (v_mfma_f32_32x32x16_bf16) or on OCP E4M3 fp8 operands with per-tensor
// scales (v_mfma_f32_32x32x64_f8f6f4):
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
// gate + 128 up accumulator columns), 256 threads = 4 wave64s laid out 2 (M) x 2 (N), one
// per SIMD; each wave owns 128 x 128 outputs = 4 x 4 MFMA 32x32 blocks (256 fp32
// accumulators per lane, held in the accumulation registers).
// Staging: K steps (32 bf16 or 64 fp8 = 64 bytes of each activation row) go global -> LDS
// directly (global_load_lds_dwordx4, no register staging) into a ring of 5 LDS stages of
// 32 KB (all 160 KB of the CU's LDS): while one step is computed the next three are landing
// or in flight and the fifth stage, released by the previous step, is being refilled. One
// barrier per K step, placed inside the step: it publishes the next stage, so the next
// stage's first operand fragments are read while the current step's MFMAs still run.
// LDS layouts: the activation tile is kept [m][k] (64-byte rows) and read with
// ds_read_b128; the weight tile is kept in its memory order [k][n] (512-byte rows for bf16,
// 256 for fp8) and read with the gfx950 transposing loads ds_read_b64_tr_b16 / _b8, which
// hand each lane 4 (bf16) or 8 (fp8) consecutive k of one column. The 16-byte granules of a
// row are XOR-permuted (activation: chunk ^ ((row >> 2) & 3); bf16 weight: granule ^
// 4 * (k & 3); fp8 weight: granule ^ 2 * (k & 7)), which makes every read free of LDS bank
// conflicts; the DMA applies the permutation by choosing which source granule each lane
// fetches.
// Tiles are ordered so that each XCD (workgroups are dealt to the 8 XCDs round-robin)
// works on a compact block of 4 row tiles x n column tiles, which keeps its L2 hit rate up.
#include <type_traits>

#include "tp_internal.h"

namespace tpk {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int BM = 256, BN = 256, NTHR = 256, NSTAGE = 5;
constexpr int A_STRIDE = 64;              // bytes per activation row (one K step)
constexpr int A_BYTES = BM * A_STRIDE;    // 16384
constexpr int B_BYTES = 16384;            // one K step of the weight tile
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int A_PER_WAVE = BM * 4 / 4;    // 256 granules of 16 B = 4 DMA instructions
constexpr int B_PER_WAVE = B_BYTES / 16 / 4;
constexpr int DMA_A = 4, DMA_B = 4;

// Operand layouts of the bf16 tiles. LAY_NN: A [M, K] with K contiguous, B [K, N] with N
// contiguous. LAY_NT: B is given as B^T [N, K] (K contiguous): its tile holds 256 columns x one
// K step of 64 bytes each, i.e. the activation tile's shape, so it is staged and read like one.
// LAY_TN: A is given as A^T [K, M] (M contiguous): its tile holds one K step of 512-byte rows,
// the weight tile's shape, and is staged and read (with the transposing LDS reads) like one.
// The backward products use them to read W and X in place instead of transposed copies.
constexpr int LAY_NN = 0, LAY_NT = 1, LAY_TN = 2;
// element offsets of K step k0 from the tile's first element of A and of B
template <int LAY>
__device__ __forceinline__ int64_t a_kstep(int64_t k0, int64_t lda) { return LAY == LAY_TN ? k0 * lda : k0; }
template <int LAY>
__device__ __forceinline__ int64_t b_kstep(int64_t k0, int64_t ldb) { return LAY == LAY_NT ? k0 : k0 * ldb; }

// Operand format: element type, K per step, elements per 16-byte granule, weight row bytes
template <bool F8>
struct Fmt;
template <>
struct Fmt<false> {   // bf16
    typedef uint16_t E;
    static constexpr int BK = 32, EPG = 8, B_STRIDE = 512, GPR = 32;
    __device__ static int swz(int k) { return 4 * (k & 3); }
};
template <>
struct Fmt<true> {    // OCP E4M3
    typedef uint8_t E;
    static constexpr int BK = 64, EPG = 16, B_STRIDE = 256, GPR = 16;
    __device__ static int swz(int k) { return 2 * (k & 7); }
};

// byte offset of logical 16-byte chunk c (0..3) of activation row r
__device__ __forceinline__ int a_lds(int r, int c) { return r * A_STRIDE + ((c ^ ((r >> 2) & 3)) << 4); }
// byte offset of logical 16-byte granule g of weight row k
template <bool F8>
__device__ __forceinline__ int b_lds(int k, int g) {
    return k * Fmt<F8>::B_STRIDE + ((g ^ Fmt<F8>::swz(k)) << 4);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
// OCP E4M3 code of f: nearest value, ties to even (the conversion instruction), with
// magnitudes past 448 saturated first (the instruction alone would give NaN); NaN stays NaN
__device__ __forceinline__ uint8_t f32_to_e4m3(float f) {
    f = f > 448.0f ? 448.0f : (f < -448.0f ? -448.0f : f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.0f, 0, false) & 0xFF);
}

template <bool F8>
struct Geom {
    typedef typename Fmt<F8>::E E;
    const E* A;    // [M, K] row-major, lda
    const E* B1;   // [K, N] row-major, ldb
    const E* B2;   // second weight of the dual (gate/up) form, else unused
    int64_t M, N, K, lda, ldb;
    int64_t zrow = -1;   // a row of A past M whose K elements are zero (LAY_NN), or -1
};

// Per-lane source offsets of one wave's share of a stage (fixed for the whole K loop; only
// the K offset moves), in elements relative to the tile's base pointers. Wave w fills
// activation rows 64w..64w+63 and a quarter of the weight rows, 4 DMA instructions of 64
// granules each; LDS granule G holds the logical granule that the XOR permutation maps to
// it. Every lane of every instruction loads an in-bounds address, so each wave issues
// exactly DMA_A + DMA_B loads per stage and vmcnt counts stay exact: rows past M and
// columns past N fetch a harmless valid address (row 0 / column n0), and granules past K
// fetch K chunk 0 and are zeroed after they land.
struct DmaPlan {
    int32_t a_off[DMA_A];   // row * lda + EPG * chunk
    int64_t b_off[DMA_B];   // k row * ldb + column, relative to the first weight (dual: the
                            // second weight's granules carry the pointer difference)
};

// geometry of LDS granule i*64+lane of this wave: activation row and logical chunk
__device__ __forceinline__ void a_granule(int wave, int i, int lane, int& row, int& c) {
    const int G = wave * A_PER_WAVE + i * 64 + lane;
    row = G >> 2;
    c = (G & 3) ^ ((row >> 2) & 3);
}
// weight k row and logical granule
template <bool F8>
__device__ __forceinline__ void b_granule(int wave, int i, int lane, int& row, int& g) {
    const int G = wave * B_PER_WAVE + i * 64 + lane;
    row = G / Fmt<F8>::GPR;
    g = (G % Fmt<F8>::GPR) ^ Fmt<F8>::swz(row);
}

template <bool DUAL, bool F8>
__device__ __forceinline__ int64_t b_offset(const Geom<F8>& g, int64_t n0, int row, int gr) {
    constexpr int HALF = Fmt<F8>::GPR / 2, EPG = Fmt<F8>::EPG;
    int64_t col, extra = 0;
    if (DUAL) {
        col = n0 + (int64_t)(gr % HALF) * EPG;
        if (gr >= HALF) extra = g.B2 - g.B1;
    } else {
        col = n0 + (int64_t)gr * EPG;
    }
    if (col >= g.N) {
        col = n0;
        extra = 0;
    }
    return extra + (int64_t)row * g.ldb + col;
}

template <bool DUAL, bool F8, int LAY = LAY_NN>
__device__ __forceinline__ void make_plan(DmaPlan& p, const Geom<F8>& g, int64_t m0, int64_t n0,
                                          int wave, int lane) {
    static_assert(LAY == LAY_NN || (!DUAL && !F8), "transposed operands: single bf16/fp16 weight only");
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
        int row, c;
        if constexpr (LAY == LAY_TN) {   // row = k, c = granule of 8 rows m (columns past M: the first)
            b_granule<false>(wave, i, lane, row, c);
            p.a_off[i] = (int32_t)(row * g.lda + (m0 + 8 * c < g.M ? 8 * c : 0));
        } else {
            a_granule(wave, i, lane, row, c);
            // rows past M load the zero row when there is one (zero operands draw less power than
            // a copy of a real row), else the tile's first row
            const int64_t stand_in = g.zrow >= 0 ? g.zrow - m0 : 0;
            p.a_off[i] = (int32_t)((m0 + row < g.M ? row : stand_in) * g.lda + Fmt<F8>::EPG * c);
        }
    }
#pragma unroll
    for (int i = 0; i < DMA_B; ++i) {
        int row, gr;
        if constexpr (LAY == LAY_NT) {   // row = output column n, gr = chunk of 8 k
            a_granule(wave, i, lane, row, gr);
            p.b_off[i] = (n0 + row < g.N ? row : 0) * g.ldb + 8 * gr;
        } else {
            b_granule<F8>(wave, i, lane, row, gr);
            p.b_off[i] = b_offset<DUAL, F8>(g, n0, row, gr);
        }
    }
}

// One 16-byte global -> LDS transfer per lane; the lanes of a wave fill 64 consecutive
// granules starting at LDS byte address `lds` (wave-uniform). Written as a volatile asm
// statement with no register outputs: the compiler then neither reorders it against other
// memory accesses nor adds its own vmcnt waits before LDS reads (it cannot tell which stage a
// DMA writes), and the kernel keeps the exact per-stage vmcnt accounting itself. The LDS
// address is a plain 32-bit offset carried in scalar registers (a generic pointer would need
// a null check per transfer to become one).
__device__ __forceinline__ void dma16(const void* src, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(src) : "memory", "m0");
}

// LDS byte address of a __shared__ buffer (a link-time constant)
__device__ __forceinline__ unsigned lds_addr(const unsigned char* p) {
    return (unsigned)(uintptr_t)((const __attribute__((address_space(3))) unsigned char*)(p));
}

// Issue this wave's DMA_A + DMA_B loads for the K step starting at k0 into `stage`. a_base and
// b_base are the tile's first elements of A and B in their layout.
template <bool DUAL, bool F8, int LAY = LAY_NN>
__device__ __forceinline__ void issue_stage(unsigned stage, const DmaPlan& p, const Geom<F8>& g,
                                            const typename Fmt<F8>::E* a_base,
                                            const typename Fmt<F8>::E* b_base, int64_t m0, int64_t n0,
                                            int64_t k0, int wave, int lane) {
    constexpr int BK = Fmt<F8>::BK, EPG = Fmt<F8>::EPG;
    const unsigned a_dst = stage + wave * A_PER_WAVE * 16;
    const unsigned b_dst = stage + A_BYTES + wave * B_PER_WAVE * 16;
    if (k0 + BK <= g.K) {
        const auto* a_k = a_base + a_kstep<LAY>(k0, g.lda);
        const auto* b_k = b_base + b_kstep<LAY>(k0, g.ldb);
#pragma unroll
        for (int i = 0; i < DMA_A; ++i) dma16(a_k + p.a_off[i], a_dst + i * 1024);
#pragma unroll
        for (int i = 0; i < DMA_B; ++i) dma16(b_k + p.b_off[i], b_dst + i * 1024);
        return;
    }
    // partial final step: granules past K fetch K chunk 0 / row 0 (zeroed once landed)
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
        int row, c;
        if constexpr (LAY == LAY_TN) {
            b_granule<false>(wave, i, lane, row, c);
            if (k0 + row >= g.K) row = 0;
            if (m0 + 8 * c >= g.M) c = 0;
            dma16(a_base + (k0 + row) * g.lda + 8 * c, a_dst + i * 1024);
        } else {
            a_granule(wave, i, lane, row, c);
            if (k0 + EPG * c >= g.K) c = 0;
            if (m0 + row >= g.M) row = 0;
            dma16(a_base + k0 + (int64_t)row * g.lda + EPG * c, a_dst + i * 1024);
        }
    }
#pragma unroll
    for (int i = 0; i < DMA_B; ++i) {
        int row, gr;
        if constexpr (LAY == LAY_NT) {
            a_granule(wave, i, lane, row, gr);
            if (k0 + 8 * gr >= g.K) gr = 0;
            if (n0 + row >= g.N) row = 0;
            dma16(b_base + k0 + (int64_t)row * g.ldb + 8 * gr, b_dst + i * 1024);
        } else {
            b_granule<F8>(wave, i, lane, row, gr);
            if (k0 + row >= g.K) row = 0;
            dma16(b_base + k0 * g.ldb + b_offset<DUAL, F8>(g, n0, row, gr), b_dst + i * 1024);
        }
    }
}

// After a partial final K step has landed: zero this wave's granules that lie past K.
template <bool F8, int LAY = LAY_NN>
__device__ __forceinline__ void zero_tail(unsigned char* stage, const Geom<F8>& g, int64_t k0,
                                          int wave, int lane) {
    unsigned char* a_dst = stage + wave * A_PER_WAVE * 16;
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
        int row, c;
        bool past;
        if constexpr (LAY == LAY_TN) {
            b_granule<false>(wave, i, lane, row, c);
            past = k0 + row >= g.K;
        } else {
            a_granule(wave, i, lane, row, c);
            past = k0 + Fmt<F8>::EPG * c >= g.K;
        }
        if (past) *reinterpret_cast<u32x4*>(a_dst + i * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    unsigned char* b_dst = stage + A_BYTES + wave * B_PER_WAVE * 16;
#pragma unroll
    for (int i = 0; i < DMA_B; ++i) {
        int row, gr;
        bool past;
        if constexpr (LAY == LAY_NT) {
            a_granule(wave, i, lane, row, gr);
            past = k0 + 8 * gr >= g.K;
        } else {
            b_granule<F8>(wave, i, lane, row, gr);
            past = k0 + row >= g.K;
        }
        if (past) *reinterpret_cast<u32x4*>(b_dst + i * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
}

// wait until at most n DMA instructions of this wave are outstanding (vmcnt(n))
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS column of the j-th 32-wide block of wave wn
template <bool DUAL>
__device__ __forceinline__ int b_col_of(int j, int wn) {
    if (DUAL) return (j < 2) ? (wn * 64 + j * 32) : (128 + wn * 64 + (j - 2) * 32);
    return wn * 128 + j * 32;
}

// ---- bf16 operand fragments ---------------------------------------------------------

// 8 consecutive k (rows ks*16 + 8*(lane/32) ..) of column col0 + lane%32 of the weight tile:
// two transposing reads, each giving 4 k of one column to every lane of a 16-lane group.
__device__ __forceinline__ bf16x8 read_b_frag(const unsigned char* Bs, int ks, int col0, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const int row = ks * 16 + 8 * (g >> 1) + (r >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (r & 3);
    const int gr = col >> 3, within = (col & 7) * 2;
    // rows row and row+4 have the same (row & 3), hence the same permutation
    const lds_u8* base = (const lds_u8*)(Bs) + b_lds<false>(row, gr) + within;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * 512));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
}

struct Frags {
    bf16x8 a[4];
    bf16x8 b[4];
};

// Pieces of the operand fragments of 16-deep K slice ks for wave (wm, wn), so that they can
// be interleaved one by one with MFMAs: piece 0..3 = activation block i (ds_read_b128),
// piece 4..7 = weight block j (two ds_read_b64_tr_b16).
// (LAY_NT: the weight block is read like an activation block; LAY_TN: the activation block is
// read with the weight tile's transposing reads.)
template <bool DUAL, int LAY = LAY_NN>
__device__ __forceinline__ void read_piece(Frags& f, int piece, const unsigned char* stage, int ks,
                                           int wm, int wn, int lane) {
    const int r32 = lane & 31, hi = lane >> 5;
    if (piece < 4) {
        if constexpr (LAY == LAY_TN)
            f.a[piece] = read_b_frag(stage, ks, wm * 128 + piece * 32, lane);
        else
            f.a[piece] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(stage + a_lds(wm * 128 + piece * 32 + r32, ks * 2 + hi)));
    } else {
        if constexpr (LAY == LAY_NT)
            f.b[piece - 4] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(stage + A_BYTES +
                                                        a_lds(b_col_of<DUAL>(piece - 4, wn) + r32, ks * 2 + hi)));
        else
            f.b[piece - 4] = read_b_frag(stage + A_BYTES, ks, b_col_of<DUAL>(piece - 4, wn), lane);
    }
}

template <bool DUAL, int LAY = LAY_NN>
__device__ __forceinline__ void read_frags(Frags& f, const unsigned char* stage, int ks, int wm,
                                           int wn, int lane) {
#pragma unroll
    for (int q = 0; q < 8; ++q) read_piece<DUAL, LAY>(f, q, stage, ks, wm, wn, lane);
}

// F16: the 16-bit operands are IEEE half values (same LDS layout and fragments as bf16)
template <bool F16>
__device__ __forceinline__ void mfma1(f32x16 (&acc)[4][4], const Frags& f, int n) {
    const int i = n >> 2, j = n & 3;
    if constexpr (F16)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, f.a[i]),
                                                           __builtin_bit_cast(f16x8, f.b[j]), acc[i][j], 0, 0, 0);
    else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// ---- fp8 operand fragments ----------------------------------------------------------
// The 32x32x64 fp8 MFMA takes 32 bytes per lane of each operand: lane l holds row (A) or
// column (B) l % 32 at k = 32 * (l / 32) + 0..31, byte b at k offset b (the same k order for
// both operands, which is all the product needs).

// half `part` (16 bytes: k = 32*(lane/32) + 16*part ..) of activation block i
__device__ __forceinline__ u32x4 read_a8_half(const unsigned char* stage, int i, int part, int wm,
                                              int lane) {
    const int r32 = lane & 31, hi = lane >> 5;
    return *reinterpret_cast<const u32x4*>(stage + a_lds(wm * 128 + i * 32 + r32, 2 * hi + part));
}

// quarter t (8 bytes: k = 32*(lane/32) + 8t .. +7) of weight block column col0 + lane%32:
// one transposing read; lane r of a 16-lane group addresses row k0 + r/2, 8 columns from
// 8*(r%2), and lane i receives column i of those 8 rows.
__device__ __forceinline__ i32x2 read_b8_quarter(const unsigned char* Bs, int t, int col0, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const int row = 32 * (g >> 1) + 8 * t + (r >> 1);
    const int col = col0 + 16 * (g & 1) + 8 * (r & 1);
    const lds_u8* p = (const lds_u8*)(Bs) + b_lds<true>(row, col >> 4) + (col & 15);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

__device__ __forceinline__ void set_a8(i32x8& v, int part, u32x4 x) {
    v[4 * part + 0] = (int)x.x;
    v[4 * part + 1] = (int)x.y;
    v[4 * part + 2] = (int)x.z;
    v[4 * part + 3] = (int)x.w;
}
__device__ __forceinline__ void set_b8(i32x8& v, int t, i32x2 x) {
    v[2 * t + 0] = x.x;
    v[2 * t + 1] = x.y;
}

__device__ __forceinline__ void mfma8(f32x16& acc, const i32x8& a, const i32x8& b) {
    // format 0 = E4M3 for both operands; zero scale operands select the unscaled instruction
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}

#define TP_FENCE() __builtin_amdgcn_sched_barrier(0)

// row of accumulator register r of block i for a lane in half `hi` (MFMA 32x32 layout)
__device__ __forceinline__ int acc_row(int i, int r, int hi) {
    return i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
}

// ---- epilogues ----------------------------------------------------------------------
// An epilogue turns one accumulator row block of a wave (32 rows) into outputs. The values go
// through a wave-private LDS tile first: in the MFMA layout a lane holds one column of 4
// consecutive rows, so direct stores would be 2- or 4-byte scatters (one store instruction per
// register); from the tile, every lane stores 16-byte chunks of whole rows (1 KB per
// instruction). EPI_LDS bytes of LDS per wave.
constexpr int EPI_LDS = 32 * 544;
static_assert(EPI_LDS <= STAGE_BYTES, "an epilogue tile must fit in one stage");

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Store ROWS x CHUNKS 16-byte chunks of the tile (row pitch PITCH) to dest(r, c) (nullptr =
// skip); RMW adds the fp32 chunk to what is in memory (accumulating fp32 epilogue); NT stores
// nontemporally (the fp32 partial outputs, which nothing in the kernel reads back: they then
// displace fewer operand lines from the L2; attn7b_tp4's O GEMM 90 -> 84 us).
template <int ROWS, int CHUNKS, int PITCH, bool RMW = false, class Dest, bool NT = false>
__device__ __forceinline__ void flush_tile(const unsigned char* lds, Dest dest, int lane) {
    wave_lds_sync();
#pragma unroll
    for (int idx = lane; idx < ROWS * CHUNKS; idx += 64) {
        const int r = idx / CHUNKS, c = idx % CHUNKS;
        unsigned char* d = dest(r, c);
        if (!d) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * PITCH + 16 * c);
        if (RMW) {
            const f32x4 old = *reinterpret_cast<const f32x4*>(d);
            *reinterpret_cast<f32x4*>(d) = old + __builtin_bit_cast(f32x4, v);
        } else if constexpr (NT) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(d));
        } else {
            *reinterpret_cast<u32x4*>(d) = v;
        }
    }
    wave_lds_sync();   // the tile is free for the next row block
}

// KIND: 0 bf16, 1 fp16, 2 fp32 overwrite, 3 fp32 +=, 4 OCP E4M3 code of v * (1 / out_div).
// Every accumulator is first multiplied by `scale` (the product of the per-tensor operand
// scales of fp8 operands; 1 for bf16).
// NT: fp32 partials stored nontemporally (outputs nothing in the step reads back soon); an output
// that the next kernel consumes right away (the MoE experts' rows, which the combine reads) keeps
// cached stores.
template <int KIND, bool RELU, bool NT = (KIND == 2)>
struct EpiStore {
    void* C;
    int64_t ldc, M, N;
    float scale, out_div;
    // accumulator row block i (acc[i][0..3]) of wave (wm, wn): 32 rows x 128 columns
    __device__ void rows(const f32x16 (&a)[4], int i, int64_t m0, int64_t n0, int wm, int wn,
                         int lane, unsigned char* lds) const {
        using T = std::conditional_t<(KIND >= 2 && KIND <= 3), float, std::conditional_t<KIND == 4, uint8_t, uint16_t>>;
        constexpr int ES = sizeof(T);
        constexpr int PITCH = 128 * ES + (ES == 4 ? 32 : 16);   // pads spread the two lane halves over the banks
        constexpr int CHUNKS = 128 * ES / 16;
        const int r32 = lane & 31, hi = lane >> 5;
        const float out_inv = 1.0f / out_div;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = a[j][r] * scale;
                if (RELU) v = v > 0.0f ? v : 0.0f;
                T t;
                if constexpr (KIND == 0) t = f32_to_bf16(v);
                else if constexpr (KIND == 1) t = f32_to_f16(v);
                else if constexpr (KIND <= 3) t = v;
                else t = f32_to_e4m3(v * out_inv);
                *reinterpret_cast<T*>(lds + acc_row(0, r, hi) * PITCH + (j * 32 + r32) * ES) = t;
            }
        const int64_t row0 = m0 + wm * 128 + i * 32, col0 = n0 + wn * 128;
        const int64_t rows_ok = M - row0, chunks_ok = (N - col0) * ES / 16;   // N is a multiple of 16 / ES
        unsigned char* base = static_cast<unsigned char*>(C) + (row0 * ldc + col0) * ES;
        auto dest = [&](int r, int c) -> unsigned char* {
            return (r < rows_ok && c < chunks_ok) ? base + ((int64_t)r * ldc) * ES + 16 * c : nullptr;
        };
        flush_tile<32, CHUNKS, PITCH, KIND == 3, decltype(dest), NT>(lds, dest, lane);
    }
    // grouped launches: this group's output rows r0 .. r0+m-1
    __device__ void shift_rows(int64_t r0, int64_t m) {
        using T = std::conditional_t<(KIND >= 2 && KIND <= 3), float, std::conditional_t<KIND == 4, uint8_t, uint16_t>>;
        C = static_cast<unsigned char*>(C) + r0 * ldc * (int64_t)sizeof(T);
        M = m;
    }
};

// h = SiLU(gate * gs) * (up * us); stored as bf16 (HK = 0), fp16 (HK = 1) or as the E4M3 code of
// h * (1 / h_scale) (HK = 2).
template <int HK>
struct EpiSwiGLU {
    void* h;   // [M, N]
    int64_t M, N;
    float gs, us, h_scale;
    // acc[i][0..1] hold gate columns, acc[i][2..3] the matching up columns: 32 rows x 64 h
    __device__ void rows(const f32x16 (&a)[4], int i, int64_t m0, int64_t n0, int wm, int wn,
                         int lane, unsigned char* lds) const {
        constexpr int ES = HK == 2 ? 1 : 2;
        constexpr int PITCH = 64 * ES + 16;
        constexpr int CHUNKS = 64 * ES / 16;
        const int r32 = lane & 31, hi = lane >> 5;
        const float h_inv = 1.0f / h_scale;   // one division per row block, not per element
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float gte = a[j][r] * gs, up = a[j + 2][r] * us;
                const float silu = gte * __builtin_amdgcn_rcpf(1.0f + __expf(-gte));   // rcp: 1 ulp
                unsigned char* t = lds + acc_row(0, r, hi) * PITCH + (j * 32 + r32) * ES;
                if constexpr (HK == 2) *t = f32_to_e4m3(silu * up * h_inv);
                else if constexpr (HK == 1) *reinterpret_cast<uint16_t*>(t) = f32_to_f16(silu * up);
                else *reinterpret_cast<uint16_t*>(t) = f32_to_bf16(silu * up);
            }
        const int64_t row0 = m0 + wm * 128 + i * 32, col0 = n0 + wn * 64;
        const int64_t rows_ok = M - row0, chunks_ok = (N - col0) * ES / 16;   // N is a multiple of 16
        unsigned char* base = static_cast<unsigned char*>(h) + (row0 * N + col0) * ES;
        flush_tile<32, CHUNKS, PITCH>(
            lds, [&](int r, int c) -> unsigned char* {
                return (r < rows_ok && c < chunks_ok) ? base + ((int64_t)r * N) * ES + 16 * c : nullptr;
            }, lane);
    }
    __device__ void shift_rows(int64_t r0, int64_t m) {
        h = static_cast<unsigned char*>(h) + r0 * N * (HK == 2 ? 1 : 2);
        M = m;
    }
};

// QKV projection epilogue: wave = one head (128 columns). q and k heads are rotated (rotate-
// half pairs (c, c+64), angles of the token's position from the table) and stored fp16 head-
// major [B, heads, S, 128] (q times ATTN_Q_SCALE); v heads are stored transposed,
// [B, hkv, 128, S]. M and S are multiples of 8, so a group of 8 consecutive rows (one
// 16-byte chunk of V^T) lies in one sequence; B*S < 2^31 (checked on the host), so token
// indexes divide in 32 bits.
struct EpiQKV {
    QKVOut o;
    int64_t M;   // B*S
    __device__ void rows(const f32x16 (&a)[4], int i, int64_t m0, int64_t n0, int wm, int wn,
                         int lane, unsigned char* lds) const {
        const int r32 = lane & 31, hi = lane >> 5;
        const int head = (int)((n0 + wn * 128) >> 7);
        const int n_heads = o.hq + 2 * o.hkv;
        if (head >= n_heads) return;
        const unsigned S = (unsigned)o.S;
        const int64_t row0 = m0 + wm * 128 + i * 32;
        const int64_t rows_ok = M - row0;
        if (head < o.hq + o.hkv) {
            constexpr int PITCH = 272;
            const bool is_q = head < o.hq;
            const int hh = is_q ? head : head - o.hq;
            const int nh = is_q ? o.hq : o.hkv;
            const float qs = is_q ? ATTN_Q_SCALE : 1.0f;
            // positions: rows come in groups of 4 consecutive tokens 8 apart; a group starts at a
            // multiple of 4 and S is a multiple of 8, so a group never wraps into the next
            // sequence, and stepping 8 rows wraps at most once. Rows past M keep a valid angle.
            unsigned s4 = (unsigned)(row0 + 4 * hi) % S;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = 4 * g + k, rl = acc_row(0, r, hi);
                    const float2* cs_row = o.rope + (int64_t)(s4 + k) * 64;
                    uint16_t* t = reinterpret_cast<uint16_t*>(lds + rl * PITCH);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int c = j * 32 + r32;   // pair (c, c + 64)
                        const float2 cs = cs_row[c];
                        const float x1 = a[j][r], x2 = a[j + 2][r];
                        t[c] = f32_to_f16((x1 * cs.x - x2 * cs.y) * qs);
                        t[c + 64] = f32_to_f16((x2 * cs.x + x1 * cs.y) * qs);
                    }
                }
                s4 += 8;
                if (s4 >= S) s4 -= S;
            }
            // 32 rows x 16 chunks: lane -> chunk lane % 16 of rows lane / 16 + 4 it
            unsigned char* dst = static_cast<unsigned char*>(is_q ? o.q : o.k);
            const unsigned tok = (unsigned)(row0 + (lane >> 4));
            unsigned b = tok / S, sq = tok - b * S;
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int r = (lane >> 4) + 4 * it;
                if (r < rows_ok)
                    *reinterpret_cast<u32x4*>(dst + ((((int64_t)b * nh + hh) * S + sq) * 128) * 2 +
                                              16 * (lane & 15)) =
                        *reinterpret_cast<const u32x4*>(lds + r * PITCH + 16 * (lane & 15));
                sq += 4;
                if (sq >= S) { sq -= S; ++b; }
            }
            wave_lds_sync();
        } else {
            // V^T tile: 128 dims x 32 tokens
            constexpr int PITCH = 80;
            const int hv = head - o.hq - o.hkv;
            // a lane holds 4 consecutive tokens of one dim per register group: 8-byte writes
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const unsigned lo = f32_to_f16(a[j][4 * g]) | ((unsigned)f32_to_f16(a[j][4 * g + 1]) << 16);
                    const unsigned hw = f32_to_f16(a[j][4 * g + 2]) | ((unsigned)f32_to_f16(a[j][4 * g + 3]) << 16);
                    *reinterpret_cast<u32x2*>(lds + (j * 32 + r32) * PITCH + acc_row(0, 4 * g, hi) * 2) = u32x2{lo, hw};
                }
            unsigned char* vt = static_cast<unsigned char*>(o.vt);
            flush_tile<128, 4, PITCH>(
                lds, [&](int d, int c) -> unsigned char* {
                    if (8 * c >= rows_ok) return nullptr;
                    const unsigned tok = (unsigned)(row0 + 8 * c), b = tok / S, s = tok - b * S;
                    return vt + ((((int64_t)b * o.hkv + hv) * 128 + d) * S + s) * 2;
                }, lane);
        }
    }
};

// the whole 128x128 accumulator of one wave through an epilogue
template <class Epi>
__device__ __forceinline__ void run_epilogue(const Epi& epi, f32x16 (&acc)[4][4], int64_t m0,
                                             int64_t n0, int wm, int wn, int lane, unsigned char* lds) {
#pragma unroll
    for (int i = 0; i < 4; ++i) epi.rows(acc[i], i, m0, n0, wm, wn, lane, lds);
}

// Logical tile L -> (row tile, column tile): groups of 4 row tiles, row fastest.
__device__ __forceinline__ void tile_of(int L, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int GM = 4;
    const int group = L / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = (tiles_m - first_m < GM) ? tiles_m - first_m : GM;
    const int r = L - group * GM * tiles_n;
    tm = first_m + r % gm;
    tn = r / gm;
}

// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8). Give XCD x a
// contiguous range of the first G logical tiles, so the tiles resident on one XCD share 4
// activation row blocks and few weight column blocks.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
    const int x = bid & 7, idx = bid >> 3, q = G >> 3, rem = G & 7;
    return x * q + (x < rem ? x : rem) + idx;
}

template <bool F8>
__device__ __forceinline__ bool k0_full(const Geom<F8>& g, int64_t k0) { return k0 + Fmt<F8>::BK <= g.K; }

// Wait until this wave's DMA for a stage has landed while the `ops` DMA instructions it issued
// after that stage's may still be in flight, zero its granules past K if it is the partial
// final step, then barrier: after it the stage is readable by every wave.
template <bool F8, int LAY = LAY_NN>
__device__ __forceinline__ void publish(unsigned char* stage, int ops, const Geom<F8>& g,
                                        int64_t k0, int wave, int lane) {
    constexpr int GRP = DMA_A + DMA_B;
    if (ops >= 3 * GRP) wait_vm<3 * GRP>();
    else if (ops >= 2 * GRP + DMA_A) wait_vm<2 * GRP + DMA_A>();
    else if (ops >= 2 * GRP) wait_vm<2 * GRP>();
    else if (ops >= GRP + DMA_A) wait_vm<GRP + DMA_A>();
    else if (ops >= GRP) wait_vm<GRP>();
    else if (ops >= DMA_A) wait_vm<DMA_A>();
    else wait_vm<0>();
    if (k0 + Fmt<F8>::BK > g.K) {
        wait_vm<0>();
        zero_tail<F8, LAY>(stage, g, k0, wave, lane);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS traffic done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// DMA instructions this wave issued after those of stage kt+1 and before publishing it: the
// stages kt+2 and kt+3 that exist, plus `refill_ops` of step kt+4
__device__ __forceinline__ int ops_after_next(int kt, int nk, int refill_ops) {
    constexpr int GRP = DMA_A + DMA_B;
    const int last = nk - 1 < kt + 3 ? nk - 1 : kt + 3;
    return GRP * (last - (kt + 1)) + refill_ops;
}

// One bf16 K step kt on stage `cur` (slice-0 fragments already in f0). Five LDS stages: while
// step kt is computed, kt+1 has landed or is landing, kt+2 and kt+3 are in flight, and step
// kt+4 is loaded into the stage of step kt-1 (`ref`), which every wave finished reading before
// the previous step's barrier. The instruction order is pinned: slice-0 MFMAs alternate with
// the reads of slice 1 (into f1) and with this wave's activation DMA for step kt+4; stage kt+1
// is published (wait + barrier); slice-1 MFMAs then alternate with the reads of stage kt+1's
// slice 0 (into f0) and with the weight DMA for step kt+4. Splitting the step's DMA over both
// halves keeps the four waves from queueing all their DMA at the texture units at once (with
// all of it after the barrier, that queue stalled the MFMA issue for ~190 of ~1340 cycles).
// STEADY steps (every step but the last five of a tile) know at compile time that a next step
// exists, that the refill is a whole step and that two later stages are in flight, so their
// instruction stream has no branches.
template <bool DUAL, bool STEADY, bool F16, int LAY>
__device__ __forceinline__ void k_step(f32x16 (&acc)[4][4], Frags& f0, Frags& f1,
                                       unsigned char* cur, unsigned char* nxt, unsigned ref_lds, int kt, int nk,
                                       int64_t kbase, const DmaPlan& p, const Geom<false>& g,
                                       const uint16_t* a_base, const uint16_t* b_base, int64_t m0, int64_t n0,
                                       int wm, int wn, int wave, int lane) {
    constexpr int BK = Fmt<false>::BK;
    constexpr int GRP = DMA_A + DMA_B;
    const bool has_next = STEADY || kt + 1 < nk;
    const bool refill = STEADY || kt + 4 < nk;
    const int64_t k_ref = kbase + (int64_t)(kt + 4) * BK;
    // whole refill steps interleave their DMA with the MFMAs; a partial final step takes the
    // general path up front
    const bool inline_dma = STEADY || (refill && k0_full<false>(g, k_ref));
    if (refill && !inline_dma) issue_stage<DUAL, false, LAY>(ref_lds, p, g, a_base, b_base, m0, n0, k_ref, wave, lane);
    const uint16_t* a_k = a_base + a_kstep<LAY>(k_ref, g.lda);
    const uint16_t* b_k = b_base + b_kstep<LAY>(k_ref, g.ldb);
    const unsigned a_dst = ref_lds + wave * A_PER_WAVE * 16;
    const unsigned b_dst = ref_lds + A_BYTES + wave * B_PER_WAVE * 16;
    TP_FENCE();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        mfma1<F16>(acc, f0, n);
        if (n < 8) read_piece<DUAL, LAY>(f1, n, cur, 1, wm, wn, lane);
        if (inline_dma && (n & 3) == 2) dma16(a_k + p.a_off[n >> 2], a_dst + (n >> 2) * 1024);
        TP_FENCE();
    }
    if constexpr (STEADY) {
        wait_vm<2 * GRP + DMA_A>();             // stage kt+1 landed; kt+2, kt+3, kt+4 (A) may be in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    } else if (has_next) {
        publish<false, LAY>(nxt, ops_after_next(kt, nk, refill ? (inline_dma ? DMA_A : GRP) : 0), g,
                       kbase + (int64_t)(kt + 1) * BK, wave, lane);
    }
    TP_FENCE();
#pragma unroll
    for (int n = 0; n < 16; ++n) {
        mfma1<F16>(acc, f1, n);
        if (has_next && n < 8) read_piece<DUAL, LAY>(f0, n, nxt, 0, wm, wn, lane);
        if (inline_dma && (n & 3) == 2) dma16(b_k + p.b_off[n >> 2], b_dst + (n >> 2) * 1024);
        TP_FENCE();
    }
}

// One fp8 K step kt (64 deep) on stage `cur`: 16 MFMAs in row-block order (n -> block
// (n/4, n%4)). On entry a[0..2] and bc[0..3] hold the step's fragments; a[3] is read during
// the first four MFMAs. The barrier that publishes stage kt+1 (and frees `cur`) follows
// them; the remaining twelve MFMAs then alternate with the reads of stage kt+1 — its weight
// fragments into bn (the other weight buffer), its activation block i into a[i] as soon as
// the last MFMA of row block i has been issued — and with the DMA loading step kt+4 into the
// stage of step kt-1 (`ref`).
template <bool DUAL, bool STEADY>
__device__ __forceinline__ void k_step_f8(f32x16 (&acc)[4][4], i32x8 (&a)[4], i32x8 (&bc)[4],
                                          i32x8 (&bn)[4], unsigned char* cur, unsigned char* nxt, unsigned ref_lds,
                                          int kt, int nk, int64_t kbase, const DmaPlan& p,
                                          const Geom<true>& g, const uint8_t* a_base, int64_t m0,
                                          int64_t n0, int wm, int wn, int wave, int lane) {
    constexpr int BK = Fmt<true>::BK;
    constexpr int GRP = DMA_A + DMA_B;
    TP_FENCE();
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        mfma8(acc[0][n], a[0], bc[n]);
        if (n < 2) set_a8(a[3], n, read_a8_half(cur, 3, n, wm, lane));
        TP_FENCE();
    }
    const bool has_next = STEADY || kt + 1 < nk;
    const bool refill = STEADY || kt + 4 < nk;
    if constexpr (STEADY) {
        wait_vm<2 * GRP>();                     // stage kt+1 landed; kt+2, kt+3 may be in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    } else if (has_next) {
        publish<true>(nxt, ops_after_next(kt, nk, 0), g, kbase + (int64_t)(kt + 1) * BK, wave, lane);
    }
    TP_FENCE();
    // step kt+4 goes to the stage of step kt-1 (free since the previous step's barrier)
    const int64_t k_ref = kbase + (int64_t)(kt + 4) * BK;
    const bool inline_dma = STEADY || (refill && k0_full<true>(g, k_ref));
    if (refill && !inline_dma) issue_stage<DUAL, true>(ref_lds, p, g, a_base, g.B1, m0, n0, k_ref, wave, lane);
    const uint8_t* a_k = a_base + k_ref;
    const uint8_t* b_k = g.B1 + k_ref * g.ldb;
    const unsigned a_dst = ref_lds + wave * A_PER_WAVE * 16;
    const unsigned b_dst = ref_lds + A_BYTES + wave * B_PER_WAVE * 16;
    const unsigned char* nb = nxt + A_BYTES;
#pragma unroll
    for (int n = 4; n < 16; ++n) {
        mfma8(acc[n >> 2][n & 3], a[n >> 2], bc[n & 3]);
        if (has_next) {
            if (n < 12) {   // weight block (n-4)/2, quarters 2*((n-4)%2) and +1
                const int j = (n - 4) >> 1, t0 = 2 * ((n - 4) & 1);
                set_b8(bn[j], t0, read_b8_quarter(nb, t0, b_col_of<DUAL>(j, wn), lane));
                set_b8(bn[j], t0 + 1, read_b8_quarter(nb, t0 + 1, b_col_of<DUAL>(j, wn), lane));
            }
            if (n == 4 || n == 5) set_a8(a[0], n - 4, read_a8_half(nxt, 0, n - 4, wm, lane));
            if (n == 8 || n == 9) set_a8(a[1], n - 8, read_a8_half(nxt, 1, n - 8, wm, lane));
            if (n == 12 || n == 13) set_a8(a[2], n - 12, read_a8_half(nxt, 2, n - 12, wm, lane));
        }
        if (inline_dma && n >= 6 && n < 6 + DMA_A) dma16(a_k + p.a_off[n - 6], a_dst + (n - 6) * 1024);
        if (inline_dma && n >= 10 && n < 10 + DMA_B) dma16(b_k + p.b_off[n - 10], b_dst + (n - 10) * 1024);
        TP_FENCE();
    }
}

// Tail split: the first g_full tiles (whole rounds of the machine, possibly none) run whole;
// each of the remaining tiles is cut into `pieces` K ranges of piece_steps K steps, one
// workgroup each, whose accumulators go to `part` in register order; gemm_fixup_kernel then
// sums a tile's pieces in piece order and runs the epilogue.
// waves per fix-up workgroup (divides 16); single-wave workgroups spread a tile's row blocks
// over the machine (4-wave ones made the QKV fix-up 1.5-2x slower)
constexpr int FIXUP_WAVES = 1;

// Grouped launches (one launch over several independent GEMMs that share N and K, e.g. the
// experts of an MoE layer): group e multiplies activation rows row0[e] .. row0[e+1]-1 by
// weight e (b_stride elements after weight e-1) into the same output rows. Its tiles are the
// logical tiles tile0[e] .. tile0[e+1]-1, ceil(rows / BM) row tiles x tiles_n each, so the
// split plan, the XCD mapping and the fix-up run over the launch's tiles as over one grid.
constexpr int MAX_GROUPS = 32;
struct NoGroups {
    static constexpr int MODE = 0;
};
struct Groups {
    static constexpr int MODE = 1;
    int n;
    int tile0[MAX_GROUPS + 1];
    int64_t row0[MAX_GROUPS + 1];
    int64_t b_stride;
    // logical tile L of the launch -> its group (scalar, fixed-index selects: the argument
    // block is never indexed dynamically); L becomes the tile's index within the group
    __device__ __forceinline__ int locate(int& L, int tiles_n, int& tiles_m, int64_t& r0, int64_t& m) const {
        int e = 0, t0 = tile0[0], t1 = tile0[1];
        int64_t a = row0[0], b = row0[1];
#pragma unroll
        for (int j = 1; j < MAX_GROUPS; ++j)
            if (j < n && L >= tile0[j]) {
                e = j;
                t0 = tile0[j];
                t1 = tile0[j + 1];
                a = row0[j];
                b = row0[j + 1];
            }
        L -= t0;
        tiles_m = (t1 - t0) / tiles_n;
        r0 = a;
        m = b - a;
        return e;
    }
};

struct SplitArgs {
    int g_full, pieces, piece_steps;
    float* part;   // [tail tiles * pieces][4 waves][256 registers][64 lanes]
};

// Two independent GEMMs with the same K and epilogue type in one launch (the dX and dW
// products of a backward step): logical tiles below tiles0 belong to the kernel's own
// geometry, the rest to (g1, e1). One grid lets the tail split balance both.
template <bool F8, class Epi>
struct Pair {
    static constexpr int MODE = 2;
    Geom<F8> g1;
    Epi e1;
    int tiles_m1, tiles_n1, tiles0;
    __device__ __forceinline__ bool second(int& L) const {
        if (L < tiles0) return false;
        L -= tiles0;
        return true;
    }
};

// One tile (or one K piece of a split tile) of the kernel below, with operand layout LAY.
template <bool F8, bool DUAL, class Epi, bool F16, int LAY>
__device__ __forceinline__ void tile_body(const Geom<F8>& g, const Epi& epi, int tiles_m, int tiles_n,
                                          const SplitArgs& sp, int L, int q, unsigned char* st0, unsigned char* st1,
                                          unsigned char* st2, unsigned char* st3, unsigned char* st4) {
    constexpr int BK = Fmt<F8>::BK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    int tm, tn;
    tile_of(L, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * (DUAL ? BN / 2 : BN);
    const auto* a_base = LAY == LAY_TN ? g.A + m0 : g.A + m0 * g.lda;
    const auto* b_base = LAY == LAY_NT ? g.B1 + n0 * g.ldb : g.B1;
    const int nk_total = (int)((g.K + BK - 1) / BK);
    int64_t kbase = 0;
    int nk = nk_total;
    if (q >= 0) {
        const int first = (q % sp.pieces) * sp.piece_steps;
        kbase = (int64_t)first * BK;
        nk = (nk_total - first < sp.piece_steps) ? nk_total - first : sp.piece_steps;
    }

    DmaPlan p;
    make_plan<DUAL, F8, LAY>(p, g, m0, n0, wave, lane);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        // prologue: steps 0..3 in flight, publish step 0; step 4 is loaded during step 0
        const unsigned l0 = lds_addr(st0), l1 = lds_addr(st1), l2 = lds_addr(st2), l3 = lds_addr(st3),
                       l4 = lds_addr(st4);
        issue_stage<DUAL, F8, LAY>(l0, p, g, a_base, b_base, m0, n0, kbase, wave, lane);
        if (nk > 1) issue_stage<DUAL, F8, LAY>(l1, p, g, a_base, b_base, m0, n0, kbase + BK, wave, lane);
        if (nk > 2) issue_stage<DUAL, F8, LAY>(l2, p, g, a_base, b_base, m0, n0, kbase + 2 * BK, wave, lane);
        if (nk > 3) issue_stage<DUAL, F8, LAY>(l3, p, g, a_base, b_base, m0, n0, kbase + 3 * BK, wave, lane);
        publish<F8, LAY>(st0, (DMA_A + DMA_B) * ((nk - 1 < 3) ? nk - 1 : 3), g, kbase, wave, lane);

        // stage of step kt (and its LDS address); sb, sc, sd hold steps kt+1, kt+2, kt+3 and se
        // (the stage of step kt-1) receives step kt+4
        unsigned char* sa = st0;
        unsigned char* sb = st1;
        unsigned char* sc = st2;
        unsigned char* sd = st3;
        unsigned char* se = st4;
        unsigned la = l0, lb = l1, lc = l2, ld = l3, le = l4;
#define TP_ROTATE1()            \
    do {                        \
        unsigned char* t = sa;  \
        sa = sb;                \
        sb = sc;                \
        sc = sd;                \
        sd = se;                \
        se = t;                 \
        const unsigned u = la;  \
        la = lb;                \
        lb = lc;                \
        lc = ld;                \
        ld = le;                \
        le = u;                 \
    } while (0)
        if constexpr (!F8) {
            Frags f0, f1;
            read_frags<DUAL, LAY>(f0, st0, 0, wm, wn, lane);
            // steady steps: kt + 4 <= nk - 2, so step kt+1 exists, the refill (step kt+4) is
            // whole and not the tile's last step, and two stages after kt+1 are in flight
            int kt = 0;
            for (; kt < nk - 5; ++kt) {
                k_step<DUAL, true, F16, LAY>(acc, f0, f1, sa, sb, le, kt, nk, kbase, p, g, a_base, b_base, m0, n0, wm, wn, wave, lane);
                TP_ROTATE1();
            }
            for (; kt < nk; ++kt) {
                k_step<DUAL, false, F16, LAY>(acc, f0, f1, sa, sb, le, kt, nk, kbase, p, g, a_base, b_base, m0, n0, wm, wn, wave, lane);
                TP_ROTATE1();
            }
        } else {
            i32x8 a[4], b0[4], b1[4];
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int part = 0; part < 2; ++part) set_a8(a[i], part, read_a8_half(st0, i, part, wm, lane));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) set_b8(b0[j], t, read_b8_quarter(st0 + A_BYTES, t, b_col_of<DUAL>(j, wn), lane));
            // Steady steps run in pairs whose second step swaps the roles of the two weight
            // fragment buffers (no copies; the branch-free steady step leaves room for both in
            // the register file); the remaining steps run one at a time and move the next
            // step's weight fragments into b0 (32 register moves).
            int kt = 0;
            for (; kt + 1 < nk - 5; kt += 2) {   // steady steps in pairs: the weight buffers swap by name
                k_step_f8<DUAL, true>(acc, a, b0, b1, sa, sb, le, kt, nk, kbase, p, g, a_base, m0, n0, wm, wn, wave, lane);
                k_step_f8<DUAL, true>(acc, a, b1, b0, sb, sc, la, kt + 1, nk, kbase, p, g, a_base, m0, n0, wm, wn, wave, lane);
                TP_ROTATE1();
                TP_ROTATE1();
            }
            for (; kt < nk - 5; ++kt) {   // steady steps, as in the bf16 loop
                k_step_f8<DUAL, true>(acc, a, b0, b1, sa, sb, le, kt, nk, kbase, p, g, a_base, m0, n0, wm, wn, wave, lane);
                TP_ROTATE1();
#pragma unroll
                for (int j = 0; j < 4; ++j) b0[j] = b1[j];
            }
            for (; kt < nk; ++kt) {
                k_step_f8<DUAL, false>(acc, a, b0, b1, sa, sb, le, kt, nk, kbase, p, g, a_base, m0, n0, wm, wn, wave, lane);
                TP_ROTATE1();
#pragma unroll
                for (int j = 0; j < 4; ++j) b0[j] = b1[j];
            }
        }
#undef TP_ROTATE1
    }
    if (q < 0) {
        __syncthreads();   // every wave is done with the stages; each now uses one as its tile
        unsigned char* tile = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
        run_epilogue(epi, acc, m0, n0, wm, wn, lane, tile);
        return;
    }
    float* dst = sp.part + ((int64_t)q * 4 + wave) * (256 * 64) + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[((i * 4 + j) * 16 + r) * 64] = acc[i][j][r];
}


// F16 (with F8 false): fp16 operands instead of bf16. LAY: operand layout of the tiles; a Pair
// launch's second GEMM uses LAY1.
template <bool F8, bool DUAL, class Epi, class Grp, bool F16 = false, int LAY = LAY_NN, int LAY1 = LAY_NN>
__global__ __launch_bounds__(NTHR, 1) void gemm_mfma_kernel(Geom<F8> g, Epi epi, int tiles_m,
                                                            int tiles_n, SplitArgs sp, Grp gr) {
    __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st3[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char st4[STAGE_BYTES];
    const int bid = (int)blockIdx.x;
    int L, q = -1;
    if (bid < sp.g_full) {
        L = xcd_remap(bid, sp.g_full);
    } else {
        // tail pieces, dealt piece-major so that each XCD takes one K piece of a contiguous run
        // of tail tiles (rows and columns its L2 shares) instead of one piece of tiles spread
        // over every column; q = tile * pieces + piece indexes the partial buffer either way
        q = bid - sp.g_full;
        if ((sp.g_full & 7) == 0) {
            const int n = (int)gridDim.x - sp.g_full, tail = n / sp.pieces;
            const int v = xcd_remap(q, n);
            q = (v % tail) * sp.pieces + v / tail;
        }
        L = sp.g_full + q / sp.pieces;
    }
    bool second = false;
    if constexpr (Grp::MODE == 2) {
        if (gr.second(L)) {
            second = true;
            g = gr.g1;
            epi = gr.e1;
            tiles_m = gr.tiles_m1;
            tiles_n = gr.tiles_n1;
        }
    }
    if constexpr (Grp::MODE == 1) {
        int64_t r0, m;
        const int e = gr.locate(L, tiles_n, tiles_m, r0, m);
        g.A += r0 * g.lda;
        if (g.zrow >= 0) g.zrow -= r0;
        g.B1 += e * gr.b_stride;
        if constexpr (DUAL) g.B2 += e * gr.b_stride;
        g.M = m;
        epi.shift_rows(r0, m);
    }
    if constexpr (LAY1 != LAY) {
        if (second) {
            tile_body<F8, DUAL, Epi, F16, LAY1>(g, epi, tiles_m, tiles_n, sp, L, q, st0, st1, st2, st3, st4);
            return;
        }
    }
    tile_body<F8, DUAL, Epi, F16, LAY>(g, epi, tiles_m, tiles_n, sp, L, q, st0, st1, st2, st3, st4);
}

// One wave per (split tile, wave of the tile, accumulator row block i): sum the tile's
// pieces in piece order, then that row block's epilogue. 16 single-wave workgroups per tile
// keep the partial reads spread over the machine.
template <bool DUAL, class Epi, class Grp>
__global__ __launch_bounds__(64 * FIXUP_WAVES) void gemm_fixup_kernel(Epi epi, int tiles_m, int tiles_n,
                                                                      SplitArgs sp, Grp gr) {
    __shared__ __attribute__((aligned(16))) unsigned char tile[FIXUP_WAVES * EPI_LDS];
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * FIXUP_WAVES + (int)(threadIdx.x >> 6);   // (tile, wave, i)
    const int t = gw >> 4, wave = (gw >> 2) & 3, i = gw & 3;
    const int wm = wave & 1, wn = wave >> 1;
    int L = sp.g_full + t;
    if constexpr (Grp::MODE == 2) {
        if (gr.second(L)) {
            epi = gr.e1;
            tiles_m = gr.tiles_m1;
            tiles_n = gr.tiles_n1;
        }
    }
    if constexpr (Grp::MODE == 1) {
        int64_t r0, m;
        gr.locate(L, tiles_n, tiles_m, r0, m);
        epi.shift_rows(r0, m);
    }
    int tm, tn;
    tile_of(L, tiles_m, tiles_n, tm, tn);
    f32x16 a[4];
    const float* src = sp.part + ((int64_t)t * sp.pieces * 4 + wave) * (256 * 64) + i * (64 * 64) + lane;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) a[j][r] = src[(j * 16 + r) * 64];
    for (int pc = 1; pc < sp.pieces; ++pc) {
        const float* s2 = src + (int64_t)pc * 4 * (256 * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) a[j][r] += s2[(j * 16 + r) * 64];
    }
    epi.rows(a, i, (int64_t)tm * BM, (int64_t)tn * (DUAL ? BN / 2 : BN), wm, wn, lane,
             tile + (threadIdx.x >> 6) * EPI_LDS);
}

// Workspace sizes are planned for gfx950's 256 compute units, so the size queries (and the
// argument checks that use them) make no HIP call. A launch plans with the CU count of the
// stream's device; if that plan needs more workspace than was given, its tiles all run whole.
constexpr int PLAN_CU = 256;

int cu_count_of(hipStream_t s) {
    static int cached[64] = {};
    int dev = -1;
    if (!s || hipStreamGetDevice(s, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess) return PLAN_CU;
    }
    if (dev < 0 || dev >= 64) return PLAN_CU;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = PLAN_CU;
        cached[dev] = n;
    }
    return cached[dev];
}

// How a grid of G tiles (nk K steps each) is cut: full tiles for whole rounds of the machine,
// the rest split into pieces so that the last round is filled.
// The tail (the tiles past the last full round, or the whole grid if it is smaller than the
// machine) is cut into p = 2..4 pieces (each keeping >= 2 K steps) when that shortens the
// tail by more than the fix-up pass costs. In K-step times: the tail takes nk tile steps
// unsplit and nk * ceil(tail*p/n_cu)/p split; every piece costs its 256 KB of fp32 partials
// written and read back, ~0.1 us at the streaming bandwidth, against ~0.75 us per K step
// (~1300 cycles at the power-limited clock), i.e. ~0.14 step per piece spread over the
// machine. Examples on 256 units: the 7B TP=4 gate/up grid (352 tiles, tail 96, nk 128) -> 2
// pieces; a grid of 160 tiles with nk 256 (70B TP=8 QKV) -> 3 pieces (two rounds of thirds);
// a grid of 176 tiles with nk 128 (the 7B MLP down shard's backward) stays whole: 4 pieces
// would save a quarter tile (32 steps) but cost ~98 steps of fix-up.
SplitArgs plan_split(int64_t G, int nk, int n_cu) {
    SplitArgs sp{(int)G, 1, nk, nullptr};
    const int64_t full = (G / n_cu) * n_cu;
    const int64_t tail = G - full;
    if (tail == 0) return sp;
    constexpr double FIXUP_STEPS_PER_PIECE = 0.14;
    int pieces = 1;
    double best = (double)nk;   // tail duration in K steps, unsplit
    for (int p = 2; p <= 4 && nk >= 2 * p; ++p) {
        const double t = (double)nk * (double)((tail * p + n_cu - 1) / n_cu) / p +
                         FIXUP_STEPS_PER_PIECE * (double)(tail * p);
        if (t < best - 1e-9) {
            best = t;
            pieces = p;
        }
    }
    if (pieces < 2) return sp;
    sp.g_full = (int)full;
    sp.pieces = pieces;
    sp.piece_steps = (nk + pieces - 1) / pieces;
    return sp;
}

template <bool DUAL>
void tiles_of(int64_t M, int64_t N, int64_t& tiles_m, int64_t& tiles_n) {
    tiles_m = (M + BM - 1) / BM;
    tiles_n = (N + (DUAL ? BN / 2 : BN) - 1) / (DUAL ? BN / 2 : BN);
}

size_t split_bytes_of(int64_t M, int64_t N, int64_t K, bool dual, int bk) {
    int64_t tm, tn;
    if (dual) tiles_of<true>(M, N, tm, tn);
    else tiles_of<false>(M, N, tm, tn);
    const SplitArgs sp = plan_split(tm * tn, (int)((K + bk - 1) / bk), PLAN_CU);
    if (sp.pieces < 2) return 0;
    return (size_t)(tm * tn - sp.g_full) * sp.pieces * 4 * 256 * 64 * sizeof(float);
}

// ws may be NULL (or too small): the tiles then all run whole. A grouped launch takes its
// tile count from the groups (g.M then only bounds nothing: each group sets its own).
template <bool F8, bool DUAL, class Epi, class Grp = NoGroups, bool F16 = false, int LAY = LAY_NN,
          int LAY1 = LAY_NN>
hipError_t launch(const Geom<F8>& g, const Epi& epi, void* ws, size_t ws_bytes, hipStream_t s,
                  const char* name, const Grp& gr = Grp{}) {
    constexpr int BK = Fmt<F8>::BK;
    int64_t tiles_m, tiles_n;
    tiles_of<DUAL>(g.M, g.N, tiles_m, tiles_n);
    int64_t G = tiles_m * tiles_n;
    if constexpr (Grp::MODE == 1) G = gr.tile0[gr.n];
    if constexpr (Grp::MODE == 2) G = gr.tiles0 + (int64_t)gr.tiles_m1 * gr.tiles_n1;
    if (G == 0) return hipSuccess;
    const int nk = (int)((g.K + BK - 1) / BK);
    SplitArgs sp = plan_split(G, nk, cu_count_of(s));
    const size_t need = sp.pieces >= 2 ? (size_t)(G - sp.g_full) * sp.pieces * 4 * 256 * 64 * sizeof(float) : 0;
    if (sp.pieces >= 2 && (!ws || ws_bytes < need)) sp = SplitArgs{(int)G, 1, nk, nullptr};
    sp.part = static_cast<float*>(ws);
    const int64_t blocks = sp.pieces >= 2 ? sp.g_full + (G - sp.g_full) * sp.pieces : G;
    {
        ProfScope ps(name, s);
        gemm_mfma_kernel<F8, DUAL, Epi, Grp, F16, LAY, LAY1><<<(unsigned)blocks, NTHR, 0, s>>>(g, epi, (int)tiles_m,
                                                                                          (int)tiles_n, sp, gr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || sp.pieces < 2) return e;
    }
    ProfScope ps(DUAL ? "fixup_swiglu" : "fixup_gemm", s);
    gemm_fixup_kernel<DUAL, Epi, Grp><<<(unsigned)((G - sp.g_full) * 16 / FIXUP_WAVES), 64 * FIXUP_WAVES, 0, s>>>(
        epi, (int)tiles_m, (int)tiles_n, sp, gr);
    return hipGetLastError();
}

// bf16 -> fp16, 8 elements (16 bytes) per thread: the exponent range of fp16 is narrower, so
// values below 2^-14 in magnitude round to fp16 subnormals (RNE) and values past 65504 to inf
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out,
                                                          int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const u32x4 v = in[i];
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float lo = __uint_as_float(v[k] << 16), hi = __uint_as_float(v[k] & 0xffff0000u);
        o[k] = (unsigned)f32_to_f16(lo) | ((unsigned)f32_to_f16(hi) << 16);
    }
    out[i] = o;
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

size_t gemm_bf16_split_bytes(int64_t M, int64_t N, int64_t K, int dual) {
    return split_bytes_of(M, N, K, dual != 0, Fmt<false>::BK);
}

size_t gemm_f8_split_bytes(int64_t M, int64_t N, int64_t K, int dual) {
    return split_bytes_of(M, N, K, dual != 0, Fmt<true>::BK);
}

hipError_t gemm_bf16_store(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int out_kind,
                           int relu, void* ws, size_t ws_bytes, hipStream_t s) {
    Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), nullptr,
                  M, N, K, lda, ldb};
#define TP_STORE_CASE(KIND, RELU)                                                                   \
    if (out_kind == KIND && (relu != 0) == RELU)                                                    \
        return launch<false, false>(g, EpiStore<KIND, RELU>{C, ldc, M, N, 1.0f, 1.0f}, ws, ws_bytes, s, \
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

hipError_t gemm_f16_store(const void* A, const void* B, void* C, int64_t M, int64_t N,
                          int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int out_kind,
                          int relu, void* ws, size_t ws_bytes, hipStream_t s) {
    Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), nullptr,
                  M, N, K, lda, ldb};
#define TP_STORE_CASE(KIND, RELU)                                                                      \
    if (out_kind == KIND && (relu != 0) == RELU)                                                       \
        return launch<false, false, EpiStore<KIND, RELU>, NoGroups, true>(                             \
            g, EpiStore<KIND, RELU>{C, ldc, M, N, 1.0f, 1.0f}, ws, ws_bytes, s,                        \
            KIND >= 2 ? "gemm_f16_f32out" : "gemm_f16_store");
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

hipError_t gemm_f8_store(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                         int64_t lda, int64_t ldb, int64_t ldc, int out_kind, int relu, float scale,
                         float out_div, void* ws, size_t ws_bytes, hipStream_t s) {
    Geom<true> g{static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), nullptr,
                 M, N, K, lda, ldb};
#define TP_STORE_CASE(KIND, RELU)                                                                     \
    if (out_kind == KIND && (relu != 0) == RELU)                                                      \
        return launch<true, false>(g, EpiStore<KIND, RELU>{C, ldc, M, N, scale, out_div}, ws, ws_bytes, s, \
                                   KIND == 2 || KIND == 3 ? "gemm_f8_f32out" : "gemm_f8_store");
    TP_STORE_CASE(0, false)
    TP_STORE_CASE(0, true)
    TP_STORE_CASE(1, false)
    TP_STORE_CASE(1, true)
    TP_STORE_CASE(2, false)
    TP_STORE_CASE(2, true)
    TP_STORE_CASE(3, false)
    TP_STORE_CASE(4, true)
#undef TP_STORE_CASE
    return hipErrorInvalidValue;
}

hipError_t gemm_bf16_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                            int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t s, int h_f16) {
    Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bg),
                  static_cast<const uint16_t*>(Bu), M, N, K, K, N};
    if (h_f16)
        return launch<false, true>(g, EpiSwiGLU<1>{h, M, N, 1.0f, 1.0f, 1.0f}, ws, ws_bytes, s, "gemm_bf16_swiglu");
    return launch<false, true>(g, EpiSwiGLU<0>{h, M, N, 1.0f, 1.0f, 1.0f}, ws, ws_bytes, s,
                               "gemm_bf16_swiglu");
}

hipError_t gemm_f16_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                           int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t s) {
    Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bg),
                  static_cast<const uint16_t*>(Bu), M, N, K, K, N};
    return launch<false, true, EpiSwiGLU<1>, NoGroups, true>(g, EpiSwiGLU<1>{h, M, N, 1.0f, 1.0f, 1.0f}, ws,
                                                             ws_bytes, s, "gemm_f16_swiglu");
}

namespace {

// groups 0..n-1 from their row offsets (n+1 entries, relative to the launch's A and output)
Groups make_groups(const int64_t* row_offsets, int n, int64_t tiles_n, int64_t b_stride) {
    Groups gr{};
    gr.n = n;
    gr.b_stride = b_stride;
    int64_t t = 0;
    for (int e = 0; e <= n; ++e) {
        gr.row0[e] = row_offsets[e];
        gr.tile0[e] = (int)t;
        if (e < n) t += (row_offsets[e + 1] - row_offsets[e] + BM - 1) / BM * tiles_n;
    }
    return gr;
}

int64_t tiles_n_of(int64_t N, bool dual) { return (N + (dual ? BN / 2 : BN) - 1) / (dual ? BN / 2 : BN); }

}  // namespace

// Launches of at most MAX_GROUPS groups each run one after another and reuse one split
// workspace: its size is the largest launch's.
size_t gemm_bf16_grouped_split_bytes(const int64_t* row_offsets, int n_groups, int64_t N, int64_t K, int dual) {
    const int64_t tn = tiles_n_of(N, dual != 0);
    const int nk = (int)((K + Fmt<false>::BK - 1) / Fmt<false>::BK);
    size_t best = 0;
    for (int x0 = 0; x0 < n_groups; x0 += MAX_GROUPS) {
        const int n = n_groups - x0 < MAX_GROUPS ? n_groups - x0 : MAX_GROUPS;
        const int64_t G = make_groups(row_offsets + x0, n, tn, 0).tile0[n];
        const SplitArgs sp = plan_split(G, nk, PLAN_CU);
        const size_t b = sp.pieces < 2 ? 0 : (size_t)(G - sp.g_full) * sp.pieces * 4 * 256 * 64 * sizeof(float);
        best = b > best ? b : best;
    }
    return best;
}

size_t gemm_bf16_pair_split_bytes(int64_t M0, int64_t N0, int64_t M1, int64_t N1, int64_t K) {
    int64_t tm0, tn0, tm1, tn1;
    tiles_of<false>(M0, N0, tm0, tn0);
    tiles_of<false>(M1, N1, tm1, tn1);
    const int64_t G = tm0 * tn0 + tm1 * tn1;
    const SplitArgs sp = plan_split(G, (int)((K + Fmt<false>::BK - 1) / Fmt<false>::BK), PLAN_CU);
    return sp.pieces < 2 ? 0 : (size_t)(G - sp.g_full) * sp.pieces * 4 * 256 * 64 * sizeof(float);
}

hipError_t gemm_bf16_f32out_pair(const void* A0, const void* B0, float* C0, int64_t M0, int64_t N0,
                                 int64_t lda0, int64_t ldb0, int64_t ldc0, const void* A1, const void* B1,
                                 float* C1, int64_t M1, int64_t N1, int64_t lda1, int64_t ldb1, int64_t ldc1,
                                 int64_t K, void* ws, size_t ws_bytes, hipStream_t s) {
    using Epi = EpiStore<2, false>;
    Geom<false> g0{static_cast<const uint16_t*>(A0), static_cast<const uint16_t*>(B0), nullptr, M0, N0, K, lda0, ldb0};
    int64_t tm0, tn0, tm1, tn1;
    tiles_of<false>(M0, N0, tm0, tn0);
    tiles_of<false>(M1, N1, tm1, tn1);
    Pair<false, Epi> pr{Geom<false>{static_cast<const uint16_t*>(A1), static_cast<const uint16_t*>(B1), nullptr,
                                    M1, N1, K, lda1, ldb1},
                        Epi{C1, ldc1, M1, N1, 1.0f, 1.0f}, (int)tm1, (int)tn1, (int)(tm0 * tn0)};
    return launch<false, false>(g0, Epi{C0, ldc0, M0, N0, 1.0f, 1.0f}, ws, ws_bytes, s, "gemm_bf16_f32out", pr);
}

hipError_t gemm_bf16_f32out_t(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                              int64_t ldb, int64_t ldc, int b_trans, void* ws, size_t ws_bytes, hipStream_t s) {
    using Epi = EpiStore<2, false>;
    const Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), nullptr, M, N, K, lda, ldb};
    if (b_trans)
        return launch<false, false, Epi, NoGroups, false, LAY_NT>(g, Epi{C, ldc, M, N, 1.0f, 1.0f}, ws, ws_bytes, s,
                                                                   "gemm_bf16_f32out_nt");
    return launch<false, false, Epi, NoGroups, false, LAY_TN>(g, Epi{C, ldc, M, N, 1.0f, 1.0f}, ws, ws_bytes, s,
                                                               "gemm_bf16_f32out_tn");
}

hipError_t gemm_bf16_f32out_pair_tn_nt(const void* A0t, const void* B0, float* C0, int64_t M0, int64_t N0,
                                       int64_t lda0, int64_t ldb0, int64_t ldc0, const void* A1, const void* B1t,
                                       float* C1, int64_t M1, int64_t N1, int64_t lda1, int64_t ldb1, int64_t ldc1,
                                       int64_t K, void* ws, size_t ws_bytes, hipStream_t s) {
    using Epi = EpiStore<2, false>;
    Geom<false> g0{static_cast<const uint16_t*>(A0t), static_cast<const uint16_t*>(B0), nullptr, M0, N0, K, lda0, ldb0};
    int64_t tm0, tn0, tm1, tn1;
    tiles_of<false>(M0, N0, tm0, tn0);
    tiles_of<false>(M1, N1, tm1, tn1);
    Pair<false, Epi> pr{Geom<false>{static_cast<const uint16_t*>(A1), static_cast<const uint16_t*>(B1t), nullptr,
                                    M1, N1, K, lda1, ldb1},
                        Epi{C1, ldc1, M1, N1, 1.0f, 1.0f}, (int)tm1, (int)tn1, (int)(tm0 * tn0)};
    return launch<false, false, Epi, Pair<false, Epi>, false, LAY_TN, LAY_NT>(
        g0, Epi{C0, ldc0, M0, N0, 1.0f, 1.0f}, ws, ws_bytes, s, "gemm_bf16_f32out_tn_nt", pr);
}

hipError_t gemm_bf16_swiglu_grouped(const void* A, const void* Bg, const void* Bu, void* h,
                                    const int64_t* row_offsets, int n_groups, int64_t N, int64_t K, void* ws,
                                    size_t ws_bytes, hipStream_t s, int64_t zero_row) {
    const int64_t M = row_offsets[n_groups], tn = tiles_n_of(N, true);
    for (int x0 = 0; x0 < n_groups; x0 += MAX_GROUPS) {
        const int n = n_groups - x0 < MAX_GROUPS ? n_groups - x0 : MAX_GROUPS;
        const int64_t wo = (int64_t)x0 * K * N;
        Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bg) + wo,
                      static_cast<const uint16_t*>(Bu) + wo, M, N, K, K, N, zero_row};
        hipError_t e = launch<false, true>(g, EpiSwiGLU<0>{h, M, N, 1.0f, 1.0f, 1.0f}, ws, ws_bytes, s,
                                           "gemm_bf16_swiglu", make_groups(row_offsets + x0, n, tn, K * N));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t gemm_bf16_f32out_grouped(const void* A, const void* B, float* C, const int64_t* row_offsets,
                                    int n_groups, int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t s,
                                    int64_t zero_row) {
    const int64_t M = row_offsets[n_groups], tn = tiles_n_of(N, false);
    for (int x0 = 0; x0 < n_groups; x0 += MAX_GROUPS) {
        const int n = n_groups - x0 < MAX_GROUPS ? n_groups - x0 : MAX_GROUPS;
        Geom<false> g{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B) + (int64_t)x0 * K * N,
                      nullptr, M, N, K, K, N, zero_row};
        hipError_t e = launch<false, false>(g, EpiStore<2, false, false>{C, N, M, N, 1.0f, 1.0f}, ws, ws_bytes, s,
                                            "gemm_bf16_f32out", make_groups(row_offsets + x0, n, tn, K * N));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t gemm_f8_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                          int64_t N, int64_t K, float gate_scale, float up_scale, float h_scale,
                          void* ws, size_t ws_bytes, hipStream_t s) {
    Geom<true> g{static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(Bg),
                 static_cast<const uint8_t*>(Bu), M, N, K, K, N};
    return launch<true, true>(g, EpiSwiGLU<2>{h, M, N, gate_scale, up_scale, h_scale}, ws, ws_bytes, s,
                              "gemm_f8_swiglu");
}

hipError_t gemm_bf16_qkv_rope(const void* X, const void* Wqkv, int64_t H, const QKVOut& o,
                              void* ws, size_t ws_bytes, hipStream_t s) {
    const int64_t M = o.B * o.S, N = (int64_t)(o.hq + 2 * o.hkv) * 128;
    Geom<false> g{static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wqkv), nullptr,
                  M, N, H, H, N};
    return launch<false, false>(g, EpiQKV{o, M}, ws, ws_bytes, s, "gemm_bf16_qkv_rope");
}

hipError_t bf16_to_f16(const void* in, void* out, int64_t n, hipStream_t s) {
    const int64_t n8 = n / 8;
    if (n8 == 0) return hipSuccess;
    ProfScope ps("bf16_to_f16", s);
    bf16_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(static_cast<const u32x4*>(in),
                                                                     static_cast<u32x4*>(out), n8);
    return hipGetLastError();
}

hipError_t rope_table(float2* table, int64_t pos0, int64_t npos, float theta, hipStream_t s) {
    const int64_t n = npos * 64;
    ProfScope ps("rope_table", s);
    rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(table, pos0, npos, (double)theta);
    return hipGetLastError();
}

}  // namespace tpk
