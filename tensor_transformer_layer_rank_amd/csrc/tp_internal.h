// Internal declarations shared by the C-ABI front end (api.cpp) and the gfx950 kernels.
// Not part of the public interface (include/tpshard.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tpshard.h"

namespace tpk {

// ---- kernel timing hook (implemented in api.cpp) --------------------------------
// Every launcher brackets its kernel with prof_begin/prof_end; both are no-ops
// unless tp_profile_enable(1) was called.
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

struct ProfScope {
    hipStream_t s;
    ProfScope(const char* name, hipStream_t st) : s(st) { prof_begin(name, st); }
    ~ProfScope() { prof_end(s); }
};

// ---- matrix-pipe rate microbenchmark (measurement aid) --------------------------------
// n_wg workgroups of 4 waves, each wave 16 * iters v_mfma_f32_32x32x16_bf16 on register
// operands loaded from ops (8 x 256 x 16 bytes); out: n_wg * 256 fp32 checksums
hipError_t mfma_rate(const void* ops, float* out, int64_t n_wg, int64_t iters, hipStream_t s);
// n_wg workgroups each reading per_wg bytes (a multiple of 8192) of buf; out: n_wg * 256 checksums
hipError_t hbm_read(const void* buf, int64_t per_wg, int64_t n_wg, unsigned* out, hipStream_t s);

// ---- the allocation-free column linear call ------------------------------------------
// Device address of the library's static scratch array (TP_NOALLOC_SCRATCH_BYTES) on the
// device of stream s; looked up once per device.
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

// ---- exact fp32 path ---------------------------------------------------------------
// C[M, N] (ldc) = act(A[M, K] (lda) . B[K, N] (ldb)); accumulate: C += A.B.
hipError_t gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, int64_t ldc, int relu, int accumulate,
                    hipStream_t s);

// ---- bf16 MFMA path -----------------------------------------------------------------
// Workspace that lets the tiles past the last full round of the machine be split along K
// (0 when the grid needs no split). Every call below accepts ws = NULL / too small: the
// tiles then all run whole.
size_t gemm_bf16_split_bytes(int64_t M, int64_t N, int64_t K, int dual);
// out_kind for gemm_bf16_store: 0 = bf16, 1 = fp16, 2 = fp32 (overwrite), 3 = fp32 (+=)
hipError_t gemm_bf16_store(const void* A, const void* B, void* C, int64_t M, int64_t N,
                           int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int out_kind,
                           int relu, void* ws, size_t ws_bytes, hipStream_t s);
// the same on fp16 operands (fp32 accumulation, same output kinds)
hipError_t gemm_f16_store(const void* A, const void* B, void* C, int64_t M, int64_t N,
                          int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int out_kind,
                          int relu, void* ws, size_t ws_bytes, hipStream_t s);
// h[M, N] (bf16, ld = N) = SiLU(A . Bg) * (A . Bu)
// Grouped forms (the experts of an MoE layer): group e = rows row_offsets[e] ..
// row_offsets[e+1]-1 of A and of the output, times weight e ([K, N], weights contiguous);
// n_groups >= 1, row_offsets non-decreasing from 0.
// Two fp32-out GEMMs with the same K in one launch (C_i = A_i [M_i, K] . B_i [K, N_i]).
size_t gemm_bf16_pair_split_bytes(int64_t M0, int64_t N0, int64_t M1, int64_t N1, int64_t K);
hipError_t gemm_bf16_f32out_pair(const void* A0, const void* B0, float* C0, int64_t M0, int64_t N0,
                                 int64_t lda0, int64_t ldb0, int64_t ldc0, const void* A1, const void* B1,
                                 float* C1, int64_t M1, int64_t N1, int64_t lda1, int64_t ldb1, int64_t ldc1,
                                 int64_t K, void* ws, size_t ws_bytes, hipStream_t s);
// The same fp32-out GEMM with one operand given transposed: b_trans = 1: B given as Bt [N, K]
// (ldb its row stride), C = A . Bt^T; b_trans = 0: A given as At [K, M] (lda its row stride),
// C = At^T . B. M, N, K multiples of 8. Workspace as gemm_bf16_split_bytes(M, N, K, 0).
hipError_t gemm_bf16_f32out_t(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                              int64_t ldb, int64_t ldc, int b_trans, void* ws, size_t ws_bytes, hipStream_t s);
// Both in one launch (same K): C0 = A0t^T . B0 and C1 = A1 . B1t^T (the backward's dW and dX).
// Workspace as gemm_bf16_pair_split_bytes.
hipError_t gemm_bf16_f32out_pair_tn_nt(const void* A0t, const void* B0, float* C0, int64_t M0, int64_t N0,
                                       int64_t lda0, int64_t ldb0, int64_t ldc0, const void* A1, const void* B1t,
                                       float* C1, int64_t M1, int64_t N1, int64_t lda1, int64_t ldb1, int64_t ldc1,
                                       int64_t K, void* ws, size_t ws_bytes, hipStream_t s);
size_t gemm_bf16_grouped_split_bytes(const int64_t* row_offsets, int n_groups, int64_t N, int64_t K, int dual);
// zero_row: a row of A (index from A's first row, lda = K) whose K elements are zero and which
// no group covers, or -1; the rows of a group's last tile past the group's end then load it
// (zero operands) instead of a copy of a real row. (zero_row + 1) * K must stay below 2^31.
hipError_t gemm_bf16_swiglu_grouped(const void* A, const void* Bg, const void* Bu, void* h,
                                    const int64_t* row_offsets, int n_groups, int64_t N, int64_t K, void* ws,
                                    size_t ws_bytes, hipStream_t s, int64_t zero_row = -1);
hipError_t gemm_bf16_f32out_grouped(const void* A, const void* B, float* C, const int64_t* row_offsets,
                                    int n_groups, int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t s,
                                    int64_t zero_row = -1);
// h_f16: h stored as fp16 instead of bf16
hipError_t gemm_bf16_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                            int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t s, int h_f16 = 0);
// the same on fp16 operands, h stored as fp16
hipError_t gemm_f16_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                           int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t s);
// out[i] = fp16(in[i]) for n bf16 values (n a multiple of 8, 16-byte aligned buffers)
hipError_t bf16_to_f16(const void* in, void* out, int64_t n, hipStream_t s);

// ---- fp8 (OCP E4M3) MFMA path: operands are uint8 codes; every accumulator is scaled ----
size_t gemm_f8_split_bytes(int64_t M, int64_t N, int64_t K, int dual);
// C = act(scale * A . B); out_kind 0 bf16, 1 fp16, 2 fp32, 3 fp32 +=, 4 E4M3 code of
// relu(scale * A . B) / out_div (relu must be 1 for kind 4)
hipError_t gemm_f8_store(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                         int64_t lda, int64_t ldb, int64_t ldc, int out_kind, int relu, float scale,
                         float out_div, void* ws, size_t ws_bytes, hipStream_t s);
// h[M, N] (E4M3 codes, ld = N) = code(SiLU(gate_scale * A . Bg) * (up_scale * A . Bu) / h_scale)
hipError_t gemm_f8_swiglu(const void* A, const void* Bg, const void* Bu, void* h, int64_t M,
                          int64_t N, int64_t K, float gate_scale, float up_scale, float h_scale,
                          void* ws, size_t ws_bytes, hipStream_t s);

// QKV projection of a prefill with rotary embedding and head-major scatter. The queries are
// stored multiplied by ATTN_Q_SCALE = log2(e) / sqrt(128), so the attention kernel's scores
// come out in log2 units of the softmax argument (one fp16 rounding, as without the scale).
constexpr float ATTN_Q_SCALE = 1.4426950408889634f * 0.08838834764831845f;
struct QKVOut {
    void* q;        // fp16 [B, hq, S, 128], times ATTN_Q_SCALE
    void* k;        // fp16 [B, hkv, S, 128]
    void* vt;       // fp16 [B, hkv, 128, S]   (values stored transposed)
    const float2* rope;   // [S, 64] (cos, sin)
    int64_t B, S;
    int hq, hkv;
};
hipError_t gemm_bf16_qkv_rope(const void* X, const void* Wqkv, int64_t H, const QKVOut& o,
                              void* ws, size_t ws_bytes, hipStream_t s);
// rotary table [npos, 64] of (cos, sin) of (pos0 + p) * theta^(-2i/128), computed in fp64
hipError_t rope_table(float2* table, int64_t pos0, int64_t npos, float theta, hipStream_t s);

// causal flash attention over the head-major fp16 q/k/vt; out bf16 [B*S, hq*128]
hipError_t flash_attn_fwd(const void* q, const void* k, const void* vt, void* out, int64_t B,
                          int64_t S, int hq, int hkv, hipStream_t s);

// ---- decode (skinny M) path ------------------------------------------------------------
// Split-K GEMMs for M <= 64 rows: chunk partials go to `part`, then a reduce kernel sums them
// in chunk order and applies the epilogue.
size_t skinny_partials_bytes(int64_t M, int64_t N, int64_t K);
size_t skinny_swiglu_partials_bytes(int64_t M, int64_t I, int64_t H);
// kind: 0 = fp32 store (ldc), 1 = fp32 +=, 2 = bf16 store, 3 = bf16 ReLU, 5 = fp16 store,
// 6 = fp16 ReLU, 7 = fp32 ReLU; f16_in: the operands are fp16 instead of bf16
hipError_t skinny_linear(const void* A, const void* B, float* part, int64_t M, int64_t N, int64_t K,
                         int64_t lda, void* C, int64_t ldc, int kind, hipStream_t s, int f16_in = 0);
// h [M, I] = SiLU(X . Wg) * (X . Wu), bf16 operands and h, or (f16) fp16 operands and h
hipError_t skinny_swiglu(const void* X, const void* Wg, const void* Wu, float* part, void* h,
                         int64_t M, int64_t I, int64_t H, hipStream_t s, int f16 = 0);
// decode attention step of an attention shard: QKV split-K partials (workspace `part`,
// skinny_partials_bytes(B, (hq + 2 hkv) * 128, H)), then one fused kernel that reduces them,
// rotates q and k by position pos, appends k and v (bf16) at cache slot pos and attends over
// slots 0..pos; out = bf16 [B, hq * 128]
hipError_t decode_attn_step(const void* X, const void* Wqkv, float* part, int64_t B, int64_t H, int hq,
                            int hkv, int64_t pos, float theta, void* k_cache, void* v_cache, int64_t cap,
                            void* out, hipStream_t s);

// The whole decode step of a rank in four launches: attention shard (QKV + RoPE + cache append
// + attention + O partial Ya), MLP shard on the same X (Ym), and the vocabulary-split head
// (logits [B, V]; V = 0: none). B <= 64; cap, pos as for decode_attn_step.
size_t decode_step_ws_bytes(int64_t B, int64_t H, int hq, int hkv, int64_t I, int64_t V);
hipError_t decode_step(const void* X, const void* Wqkv, const void* Wo, const void* Wg, const void* Wu,
                       const void* Wd, const void* Wlm, int64_t B, int64_t H, int hq, int hkv, int64_t I,
                       int64_t V, int64_t pos, float theta, void* k_cache, void* v_cache, int64_t cap, float* Ya,
                       float* Ym, float* logits, void* ws, hipStream_t s, bool packed = false);
// W [K, N] 16-bit -> [ceil(N / 128)][K][128] (the decode kernels' strip layout)
size_t packed_strips_bytes(int64_t K, int64_t N);
hipError_t pack_strips(const void* W, int64_t K, int64_t N, void* P, hipStream_t s);

// ---- backward of a linear shard ---------------------------------------------------------
// dX [T, K] fp32 = dY [T, N] . W^T, dW [K, N] fp32 = X^T [K, T] . dY (bf16 operands; T, K, N
// multiples of 8; W and X read in place as transposed operands). Workspace: the GEMMs' tail-split
// partials.
size_t linear_backward_ws_bytes(int64_t T, int64_t K, int64_t N);
hipError_t linear_backward(const void* X, const void* W, const void* dY, float* dX, float* dW, int64_t T,
                           int64_t K, int64_t N, void* ws, hipStream_t s);

// ---- mixture of experts ------------------------------------------------------------------
// Xg[r] = X[row_token[r]] (bf16 [R, H]; out-of-range tokens give a zero row); z0[0 .. n0-1] and
// z1[0 .. n1-1] (bf16, n multiples of 8; NULL = none) are set to zero as well;
// Y[t] = sum_j gates[t, j] * Yg[token_rows[t, j]] (fp32 [T, H]; out-of-range rows skipped).
hipError_t moe_gather(const void* X, const int32_t* row_token, void* Xg, int64_t R, int64_t T, int64_t H,
                      hipStream_t s, void* z0 = nullptr, int64_t n0 = 0, void* z1 = nullptr, int64_t n1 = 0);
hipError_t moe_combine(const float* Yg, const int32_t* token_rows, const float* gates, int k, float* Y, int64_t T,
                       int64_t R, int64_t H, hipStream_t s);

// ---- merges -------------------------------------------------------------------------------
hipError_t partial_sum(const float* const* parts, int k, float* out, int64_t n, hipStream_t s);
// r = residual + ((P0 + P1) + ...) (fp32), residual_out = bf16(r),
// normed = bf16(r / sqrt(mean_row(r^2) + eps) * gamma); bf16 [T, H], H % 8 == 0, H <= 16384
hipError_t merge_rmsnorm(const float* const* parts, int k, const void* residual, const void* gamma, float eps,
                         void* residual_out, void* normed, int64_t T, int64_t H, hipStream_t s);

}  // namespace tpk
