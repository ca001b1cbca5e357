/*
 * libtpshard — one tensor-parallel rank's shard of a Transformer block, on one
 * AMD Instinct MI355X (gfx950).
 *
 * What a rank computes (sources are the pages' titles and sections):
 *   - a column-parallel linear layer: Y_r = X . W[:, cols_r], X replicated
 *     ("CUDA tensor parallel computations", 第二类 Column Parallel;
 *      "张量并行：切分 Transformer 层的分布式训练", 列切分);
 *   - a row-parallel linear layer whose output is this rank's additive
 *     contribution to the layer output: P_r = X[:, rows_r] . W[rows_r, :]
 *     ("CUDA tensor parallel computations", 第三类 Row Parallel; 行切分);
 *   - the MLP and attention blocks built from the two ("放进 Transformer";
 *     "Transformer 层的张量并行切分": MLP 块切分, 自注意力块切分);
 *   - the element-wise sum of partial outputs, i.e. the arithmetic that an
 *     all-reduce performs (第四类 跨卡通信计算). tp_partial_sum adds buffers that
 *     all live on the calling GPU; it is not a collective.
 *
 * Conventions shared by every call
 *   - Row-major everywhere. Weights are stored [in, out] (X . W orientation, as in
 *     both pages' examples). Activations are [T, H] with T = B * S tokens,
 *     sequence-major.
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or keeps a pointer; scratch space is a caller-owned
 *     workspace whose size is queried first (one call, tp_column_linear_noalloc, uses a
 *     fixed static device array instead).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream). Buffers must stay alive until the stream has finished with them.
 *   - Arguments are validated on the host before any HIP call; on failure the call
 *     returns a non-OK status, launches nothing and tp_last_error() describes why.
 *     A failed kernel launch returns TP_ERR_HIP. Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - fp32 path: any positive sizes, 4-byte aligned pointers.
 *     bf16/fp16 path: 16-byte aligned base pointers; K, N and leading dimensions
 *     multiples of 8 elements. Tails of T and N inside a tile are masked.
 *     fp8 path (TP_FP8_E4M3, OCP E4M3 codes, one byte each, with fp32 per-tensor
 *     scales): 16-byte aligned base pointers; K and N multiples of 16. The pages
 *     name no number format; E4M3 is an extension of the same layers.
 *   - Results do not depend on launch timing: repeated calls give bitwise-equal
 *     outputs (no floating-point atomics).
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 1

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
    TP_ERR_BAD_SHAPE = 2,      /* non-positive size, ld < N, uneven head grouping, ... */
    TP_ERR_BAD_DTYPE = 3,      /* dtype combination not offered by this call */
    TP_ERR_MISALIGNED = 4,     /* pointer or size breaks the alignment rules above */
    TP_ERR_WORKSPACE = 5,      /* workspace NULL or smaller than the queried size */
    TP_ERR_UNSUPPORTED = 6,    /* well-formed but not implemented (e.g. head_dim != 128) */
    TP_ERR_HIP = 7             /* the HIP runtime reported an error at launch */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1, TP_F16 = 2, TP_FP8_E4M3 = 3 } tp_dtype;
typedef enum { TP_ACT_NONE = 0, TP_ACT_RELU = 1 } tp_act;
typedef enum { TP_MLP_RELU = 0, TP_MLP_SWIGLU = 1 } tp_mlp_kind;

/* Per-tensor dequantisation scales for TP_FP8_E4M3 operands (OCP E4M3: sign, 4
 * exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest
 * magnitude 448): real value = code_value * scale. Required (non-NULL) when
 * in_dt == TP_FP8_E4M3, ignored otherwise. */
typedef struct { float x_scale; float w_scale; } tp_fp8_scales;

/*
 * tp_column_linear — column-parallel rank output Y = act(X . W_shard).
 *   ("CUDA tensor parallel computations", 第二类 Column Parallel; 第五类 局部逐元素计算
 *    for the local activation.) Also serves the vocabulary-split output layer
 *   ("张量并行：切分 Transformer 层的分布式训练", 输入与输出层): logits for this rank's
 *   vocabulary columns.
 *   X       [T, K]   in_dt          replicated input
 *   W_shard [K, N]   in_dt          this rank's columns of the full weight
 *   Y       [T, ldy] out_dt         row t of the result at Y + t*ldy; ldy >= N lets a
 *                                   rank write its slice of a full [T, N*tp] buffer
 *                                   (the concatenation happens in place).
 *   in_dt/out_dt: (F32, F32) — exact fp32 path; (BF16 or F16, BF16|F16|F32) with fp32
 *                 accumulation;
 *                 (FP8_E4M3, BF16|F16|F32) with scales q: Y = act(x_scale * w_scale *
 *                 (codes(X) . codes(W))), accumulated in fp32.
 *   16-bit and fp8 operands: K < 2^23 (else TP_ERR_UNSUPPORTED).
 *   workspace: >= tp_linear_workspace_size(T, K, N, in_dt) bytes.
 *   act: TP_ACT_NONE or TP_ACT_RELU (applied in fp32 before the output rounding).
 */
tp_status tp_column_linear(const void* X, const void* W_shard, void* Y,
                           int64_t T, int64_t K, int64_t N, int64_t ldy,
                           tp_dtype in_dt, tp_dtype out_dt, tp_act act,
                           const tp_fp8_scales* q, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * tp_row_linear_partial — row-parallel rank contribution P = X_shard . W_shard
 *   ("CUDA tensor parallel computations", 第三类 Row Parallel): the fp32 partial
 *   that a sum over ranks (all-reduce) turns into the layer output.
 *   X_shard [T, K_shard] in_dt      this rank's slice of the input features
 *   W_shard [K_shard, N] in_dt      this rank's rows of the full weight
 *   Y_partial [T, N] fp32           overwritten, or += when accumulate != 0
 *   in_dt: F32 (exact path), BF16 or F16 (fp32 accumulation), or FP8_E4M3 with scales q
 *          (P = x_scale * w_scale * (codes(X_shard) . codes(W_shard)), fp32 accumulation).
 *   16-bit and fp8 operands: K_shard < 2^23 (else TP_ERR_UNSUPPORTED).
 *   workspace: >= tp_linear_workspace_size(T, K_shard, N, in_dt) bytes (both calls).
 */
tp_status tp_row_linear_partial(const void* X_shard, const void* W_shard, float* Y_partial,
                                int64_t T, int64_t K_shard, int64_t N, tp_dtype in_dt,
                                int accumulate, const tp_fp8_scales* q, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * Workspace bytes needed by tp_column_linear / tp_row_linear_partial for these sizes
 * (K = the contraction length). Pure host arithmetic (no HIP call): the tile split is
 * planned for gfx950's 256 compute units. Two cases use it, both fp32 partials summed in
 * a fixed order (results are run-to-run identical):
 *   - the few-row (decode) regime, T <= 64: the contraction is split into chunks;
 *   - larger 16-bit / fp8 products whose 256x256 output tiles do not fill whole rounds of
 *     the compute units: the tiles past the last full round are split along K (a launch
 *     on a device with another CU count runs every tile whole if its own plan needs more
 *     than was given).
 * When it returns 0, workspace may be NULL.
 */
size_t tp_linear_workspace_size(int64_t T, int64_t K, int64_t N, tp_dtype in_dt);

/*
 * tp_mlp_shard — one rank's MLP block: column-split first layer, local activation,
 *   row-split second layer ("CUDA tensor parallel computations", 放进 Transformer:
 *   MLP 一扩一收; "张量并行：切分 Transformer 层的分布式训练", MLP 块切分).
 *   kind TP_MLP_RELU:   P = relu(X . W_gate) . W_down          (W_up must be NULL)
 *   kind TP_MLP_SWIGLU: P = (SiLU(X . W_gate) * (X . W_up)) . W_down,
 *                       SiLU(z) = z / (1 + exp(-z)), evaluated in fp32.
 *   X [T, H], W_gate/W_up [H, I_shard], W_down [I_shard, H]: in_dt (F32, BF16 or F16)
 *   Y_partial [T, H] fp32 (overwritten).
 *   h_dt: storage type of the activated intermediate h [T, I_shard], which lives
 *   only in the workspace: F32 for the F32 path; F16 for the F16 path (fp16 operands
 *   throughout, fp32 accumulation, any T); BF16 or F16 for the BF16 path. There, F16 (T > 64
 *   only, else TP_ERR_UNSUPPORTED) keeps 3 more bits of h for wide shards (h's rounding is the
 *   largest error term of the block): the down projection then runs on fp16 operands, with
 *   W_down converted to fp16 into the workspace first (exact for |w| >= 2^-14; smaller
 *   weights round to fp16 subnormals, an error below 2^-25).
 *   The gate/up pre-activations never leave registers.
 *   workspace: >= tp_mlp_workspace_size(T, H, I_shard, kind, in_dt, h_dt) bytes,
 *   16-byte aligned; contents on return are unspecified.
 */
tp_status tp_mlp_shard(const void* X, const void* W_gate, const void* W_up,
                       const void* W_down, float* Y_partial,
                       int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind,
                       tp_dtype in_dt, tp_dtype h_dt,
                       void* workspace, size_t ws_bytes, void* stream);
size_t tp_mlp_workspace_size(int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind,
                             tp_dtype in_dt, tp_dtype h_dt);

/*
 * tp_mlp_shard_fp8 — tp_mlp_shard on OCP E4M3 operands with per-tensor scales. The
 *   activated intermediate h is itself stored as E4M3 codes with the static scale
 *   h_scale (the down projection's input must be fp8 too):
 *     g = x_scale*wg_scale * (X . W_gate),  u = x_scale*wu_scale * (X . W_up)   (fp32)
 *     h = SiLU(g) * u   (TP_MLP_SWIGLU)   or   relu(g)   (TP_MLP_RELU, W_up NULL)
 *     code(h) = nearest E4M3 value to h / h_scale (fp32 division; ties to even;
 *               magnitudes past 448 saturate to +-448)
 *     P = h_scale*wd_scale * (code(h) . W_down)   fp32, overwritten
 *   X [T, H], W_gate/W_up [H, I_shard], W_down [I_shard, H]: E4M3 codes.
 *   Requires H and I_shard multiples of 16 and 16-byte aligned pointers.
 *   workspace >= tp_mlp_fp8_workspace_size(T, H, I_shard, kind) bytes, 16-byte aligned. On
 *   return its first T * I_shard bytes hold code(h), [T, I_shard] row-major (the rest is
 *   unspecified).
 */
typedef struct {
    float x_scale, w_gate_scale, w_up_scale, w_down_scale, h_scale;
} tp_fp8_mlp_scales;
tp_status tp_mlp_shard_fp8(const void* X, const void* W_gate, const void* W_up,
                           const void* W_down, float* Y_partial,
                           int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind,
                           const tp_fp8_mlp_scales* q,
                           void* workspace, size_t ws_bytes, void* stream);
size_t tp_mlp_fp8_workspace_size(int64_t T, int64_t H, int64_t I_shard, tp_mlp_kind kind);

/*
 * tp_attn_desc — shapes of one rank's attention shard (all head counts are the
 * rank's local ones). The rank holds whole heads ("张量并行：切分 Transformer 层的
 * 分布式训练", 自注意力块切分); query heads share kv heads in groups
 * ("TensorRT LLM 中的并行策略", 注意力模块): q head j reads kv head
 * floor(j * n_kv_heads / n_q_heads).
 *   B, S, H        sequences, tokens per sequence, hidden size (T = B*S rows of X);
 *                  prefill: S a multiple of 8, S <= 2^24 and T < 2^31 (else
 *                  TP_ERR_MISALIGNED / TP_ERR_UNSUPPORTED)
 *   head_dim       must be 128
 *   rope_theta     rotary base; rotate-half pairs (i, i+64), angle pos*theta^(-2i/128),
 *                  applied to q and k; pos = index in the sequence (decode: cache_len)
 *   causal         must be 1 (key position <= query position, within a sequence)
 *   k_cache, v_cache  decode only (S == 1): [B, n_kv_heads, cache_capacity, 128] in_dt,
 *                  slots < cache_len hold rotated keys / values; the call writes the
 *                  new token's rotated key and value at slot cache_len and attends to
 *                  slots 0..cache_len. NULL for prefill.
 */
typedef struct {
    int64_t B, S, H;
    int32_t n_q_heads, n_kv_heads, head_dim;
    float rope_theta;
    int32_t causal;
    void* k_cache;
    void* v_cache;
    int64_t cache_len, cache_capacity;
} tp_attn_desc;

/*
 * tp_attn_shard — one rank's attention block: QKV column projection, rotary
 *   embedding, per-head causal softmax(q k^T / sqrt(128)) v on the local heads,
 *   then the O row projection's fp32 partial ("CUDA tensor parallel computations",
 *   放进 Transformer: QKV / Attention heads / 输出投影).
 *   X      [B*S, H] in_dt (BF16)
 *   W_qkv  [H, (hq + 2*hkv)*128]: columns [Q heads | K heads | V heads], 128 each
 *   W_o    [hq*128, H]
 *   Y_partial [B*S, H] fp32 (overwritten)
 *   workspace >= tp_attn_workspace_size(desc, in_dt) bytes, 16-byte aligned.
 */
tp_status tp_attn_shard(const void* X, const void* W_qkv, const void* W_o, float* Y_partial,
                        const tp_attn_desc* desc, tp_dtype in_dt,
                        void* workspace, size_t ws_bytes, void* stream);
size_t tp_attn_workspace_size(const tp_attn_desc* desc, tp_dtype in_dt);

/*
 * tp_decode_step — one rank's whole decode step (one new token for each of B sequences) in four
 *   launches: its attention shard with the KV cache kept on the rank ("TensorRT LLM 中的并行策略",
 *   注意力模块), its MLP shard, and its slice of the vocabulary-split output layer ("张量并行：切分
 *   Transformer 层的分布式训练", 输入与输出层), all on the same input X. QKV and gate/up stream their
 *   weights in one launch, the attention launch also forms h, and O, down and the output layer
 *   share one more launch before a final reduction, so the step pays the start and end of a
 *   launch four times instead of once per layer.
 *   X [B, H] bf16, B <= 64; desc: a decode step (S == 1, k_cache / v_cache, cache_len <
 *   cache_capacity; the call appends the new token's rotated key and value at slot cache_len, as
 *   tp_attn_shard does); W_qkv, W_o as for tp_attn_shard; W_gate, W_up [H, I_shard] and W_down
 *   [I_shard, H] bf16 (SwiGLU); W_lm [H, V_shard] bf16, or NULL with V_shard = 0 (no output layer).
 *   Y_attn, Y_mlp [B, H] fp32 partials (overwritten); logits [B, V_shard] fp32.
 *   The results are those of tp_attn_shard, tp_mlp_shard and tp_column_linear (fp32 output) on the
 *   same arguments, up to the order of their fp32 split sums. H, I_shard, V_shard multiples of 8;
 *   tensors 16-byte aligned; workspace >= tp_decode_step_workspace_size(desc, I_shard, V_shard)
 *   bytes, 16-byte aligned (contents on return unspecified). Deterministic.
 */
tp_status tp_decode_step(const void* X, const void* W_qkv, const void* W_o, const tp_attn_desc* desc,
                         const void* W_gate, const void* W_up, const void* W_down, int64_t I_shard,
                         const void* W_lm, int64_t V_shard, float* Y_attn, float* Y_mlp, float* logits,
                         void* workspace, size_t ws_bytes, void* stream);
size_t tp_decode_step_workspace_size(const tp_attn_desc* desc, int64_t I_shard, int64_t V_shard);

/*
 * tp_decode_step_packed — tp_decode_step with every weight (W_qkv, W_o, W_gate, W_up, W_down,
 *   W_lm) in the strip layout that tp_pack_strips writes, each packed from the [K, N] weight that
 *   tp_decode_step would take (W_qkv from [H, (n_q_heads + 2 n_kv_heads) 128], W_o from
 *   [n_q_heads 128, H], W_gate / W_up from [H, I_shard], W_down from [I_shard, H], W_lm from
 *   [H, V_shard]); the library cannot check the packed buffers' sizes. The other arguments, the
 *   workspace size (tp_decode_step_workspace_size), the errors and the results are those of
 *   tp_decode_step, bit for bit (same kernels and sums; only the weight addresses differ). The
 *   rank's weights are streamed once per step in both forms: packed, a workgroup's K chunk of a
 *   strip is one contiguous block ("TensorRT LLM 中的并行策略", 注意力模块 and "张量并行：切分
 *   Transformer 层的分布式训练", 输入与输出层, as for tp_decode_step).
 *
 * tp_pack_strips — W [K, N] (bf16 or fp16, row-major) rearranged into 128-column strips:
 *   W_packed [ceil(N / 128)][K][128], strip s holding columns 128 s .. 128 s + 127 of every row,
 *   columns past N zero. A weight is packed once (at load time); a decode step then streams each
 *   strip as one contiguous block. W_packed: tp_packed_strips_bytes(K, N) bytes, caller-owned,
 *   must not overlap W. N a multiple of 8; K x (N rounded up to 128) at most 2^36 elements
 *   (TP_ERR_UNSUPPORTED otherwise); pointers 16-byte aligned. Asynchronous on
 *   the stream. tp_packed_strips_bytes returns 0 for shapes tp_pack_strips rejects.
 */
tp_status tp_decode_step_packed(const void* X, const void* W_qkv, const void* W_o, const tp_attn_desc* desc,
                                const void* W_gate, const void* W_up, const void* W_down, int64_t I_shard,
                                const void* W_lm, int64_t V_shard, float* Y_attn, float* Y_mlp, float* logits,
                                void* workspace, size_t ws_bytes, void* stream);
tp_status tp_pack_strips(const void* W, int64_t K, int64_t N, void* W_packed, void* stream);
size_t tp_packed_strips_bytes(int64_t K, int64_t N);

/*
 * tp_partial_sum — out = ((P_0 + P_1) + P_2) + ... + P_{k-1}, element-wise, in that
 *   order, fp32 ("CUDA tensor parallel computations", 第三类 Row Parallel: partial
 *   contributions are summed; 第四类: the all-reduce result). All buffers are on the
 *   calling GPU.
 *   partials: HOST array of k device pointers, each to n_elems floats (16-byte
 *   aligned). 1 <= k <= 16. out may alias partials[0].
 */
tp_status tp_partial_sum(const float* const* partials, int32_t k, float* out,
                         int64_t n_elems, void* stream);

/*
 * tp_merge_rmsnorm — the step after the merge of a row-parallel block: add the block
 *   output to the residual stream and normalise it for the next block. The merge is the
 *   all-reduce result ("CUDA tensor parallel computations", 第四类 跨卡通信计算); a norm
 *   reads a whole hidden row, so it runs on that merged output (same page, 第五类
 *   局部逐元素计算, on LayerNorm / RMSNorm). Per row t of T:
 *     r            = residual[t, :] + (((P_0 + P_1) + P_2) + ... + P_{k-1})[t, :]   (fp32)
 *     residual_out = bf16(r)                                         (round to nearest even)
 *     normed       = bf16(r * (1 / sqrt(mean_j r_j^2 + eps)) * gamma)
 *   (the usual RMSNorm: the pages do not print its formula).
 *   partials: HOST array of k device pointers to [T, H] fp32, 1 <= k <= 16;
 *   residual, residual_out, normed: [T, H] bf16 row-major; gamma: [H] bf16.
 *   All device buffers 16-byte aligned; H a multiple of 8 and <= 16384; T < 2^31;
 *   eps finite and >= 0 (else TP_ERR_BAD_SHAPE / TP_ERR_UNSUPPORTED / TP_ERR_MISALIGNED).
 *   residual_out may be residual (in-place update); normed must not overlap any input.
 *   No workspace; asynchronous on `stream`; deterministic (fixed reduction order).
 */
tp_status tp_merge_rmsnorm(const float* const* partials, int32_t k, const void* residual,
                           const void* gamma, float eps, void* residual_out, void* normed,
                           int64_t T, int64_t H, void* stream);

/*
 * tp_linear_backward — gradients of one rank's linear shard Y_r = X_r . W_r for the backward
 *   pass: dX = dY_r . W_r^T and dW_r = X_r^T . dY_r ("张量并行：切分 Transformer 层的分布式
 *   训练", 列切分 / 行切分, 前向与反向的通信对称). The same two products serve both splits:
 *   a column shard passes the replicated X and the gradient of its output columns, and its dX
 *   is a partial that the ranks sum (tp_partial_sum on one GPU); a row shard passes its input
 *   columns X_r and the replicated dY, and its dX is its complete slice of the input gradient.
 *   dW_r is local in both.
 *   X [T, K], W_shard [K, N], dY [T, N]: in_dt (BF16) row-major; dX [T, K] and dW [K, N] fp32
 *   (overwritten). T, K, N multiples of 8 and below 2^23; all pointers 16-byte aligned;
 *   workspace >= tp_linear_backward_workspace_size(T, K, N) bytes, 16-byte aligned (the
 *   split-K partials of the GEMMs' last round; 0 bytes, and workspace may be NULL, when both
 *   grids fill whole rounds). W and X are read in place (no transposed copies). At most 2^22
 *   output tiles of 256 x 256 in dX and dW together. fp32 accumulation; deterministic.
 */
tp_status tp_linear_backward(const void* X, const void* W_shard, const void* dY, float* dX, float* dW,
                             int64_t T, int64_t K, int64_t N, tp_dtype in_dt, void* workspace,
                             size_t ws_bytes, void* stream);
size_t tp_linear_backward_workspace_size(int64_t T, int64_t K, int64_t N);

/*
 * tp_moe_mlp_shard — one rank's fp32 partial of a top-k mixture-of-experts MLP over its local
 *   experts, each expert's weights TP-sharded like a dense MLP shard ("TensorRT LLM 中的并行
 *   策略", 混合专家 (MoE): the TP and hybrid ETP modes). The router's choice arrives as:
 *   expert_offsets: HOST array [E+1], offsets[0] = 0, non-decreasing; the R = offsets[E]
 *     dispatched rows are grouped by expert (rows offsets[e] .. offsets[e+1]-1 go to expert e);
 *   row_token: device int32 [R], the token of each row (a token outside [0, T) gives a zero row);
 *   token_rows: device int32 [T, k], the rows of each token's k slots (-1, or any index outside
 *     [0, R): an expert not on this rank); gates: device fp32 [T, k].
 *   Y_partial[t] = sum_j gates[t, j] * MLP_e(X[t]) over the valid slots, in slot order, where
 *   MLP_e(x) = (SiLU(x.W_gate[e]) * (x.W_up[e])) . W_down[e] (fp32; summed over the TP group it
 *   is the layer's MoE output, since the combine is linear).
 *   X [T, H] bf16; W_gate, W_up [E, H, I_shard], W_down [E, I_shard, H] bf16 row-major; Y_partial
 *   [T, H] fp32 (overwritten; tokens without a valid slot get 0). H, I_shard multiples of 8;
 *   1 <= E <= 1024; 1 <= k <= 16; X, weights, Y_partial 16-byte aligned; the int32/fp32
 *   routing arrays 4-byte aligned; workspace >= tp_moe_workspace_size(...) bytes, 16-byte
 *   aligned (the gathered rows, their fp32 outputs, and either h for all rows plus the GEMM
 *   split partials, with one zero row appended to the gathered rows and to h for the grouped
 *   GEMMs' padding rows, or one expert's MLP workspace). Broken rules return TP_ERR_NULL_POINTER /
 *   TP_ERR_BAD_SHAPE / TP_ERR_UNSUPPORTED / TP_ERR_MISALIGNED / TP_ERR_WORKSPACE before any
 *   launch. When an expert has more than 64 rows all experts share one grouped gate/up and one
 *   grouped down GEMM launch (per 32 experts); otherwise the experts run one after another
 *   through the weight-streaming kernels. Asynchronous on `stream`; deterministic.
 */
tp_status tp_moe_mlp_shard(const void* X, int64_t T, int64_t H, int64_t I_shard, int32_t E,
                           const void* W_gate, const void* W_up, const void* W_down,
                           const int64_t* expert_offsets, const int32_t* row_token, int32_t k,
                           const int32_t* token_rows, const float* gates, float* Y_partial,
                           void* workspace, size_t ws_bytes, void* stream);
size_t tp_moe_workspace_size(int64_t T, int64_t H, int64_t I_shard, int32_t E,
                             const int64_t* expert_offsets);

/*
 * tp_column_linear_noalloc — tp_column_linear without a workspace argument, for callers that
 *   cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 *   that forbid allocation). Same arguments, rules, results and error statuses as
 *   tp_column_linear, minus workspace/ws_bytes; it calls no allocator. Its scratch (the few-row
 *   regime's fp32 partial sums, or the split of the tiles past the last full round of the
 *   machine) is a static array of TP_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 *   runs on until the process ends:
 *     - T <= 64 needs tp_linear_workspace_size(T, K, N, in_dt) bytes of it; a call that needs more
 *       returns TP_ERR_UNSUPPORTED before any HIP call;
 *     - larger T uses the tail split only when its partials fit (otherwise every tile runs whole:
 *       the same products summed in another order, so the result can differ from
 *       tp_column_linear's in the last bits of fp32 rounding; bitwise equal when the split fits).
 *   The first call on a device looks the array's address up on that device (a HIP call that can
 *   fail with TP_ERR_HIP). All calls on one GPU share the array: calls that overlap on one GPU
 *   (other streams, other host threads) race and must be ordered by the caller. Nothing in it
 *   needs to start at zero; its contents after a call are unspecified.
 */
#define TP_NOALLOC_SCRATCH_BYTES (16u << 20)
tp_status tp_column_linear_noalloc(const void* X, const void* W_shard, void* Y,
                                   int64_t T, int64_t K, int64_t N, int64_t ldy,
                                   tp_dtype in_dt, tp_dtype out_dt, tp_act act,
                                   const tp_fp8_scales* q, void* stream);

/* Status text, thread-local detail of this thread's last non-OK status, ABI version. */
const char* tp_status_string(tp_status st);
const char* tp_last_error(void);
int tp_abi_version(void);

/*
 * Kernel timing for measurement: when enabled, the library brackets every kernel it
 * launches with a pair of HIP events on the launch stream (the events are created
 * by the library on first use). tp_profile_read synchronises those events and
 * returns the summed duration and launch count of the kernels whose name starts
 * with `prefix` ("" for all). tp_profile_reset discards the recorded pairs.
 * Off by default; at most 65536 launches are recorded between resets.
 */
tp_status tp_profile_enable(int on);
/*
 * Measurement aid (not part of the shard computation): the matrix pipe's sustained bf16 rate
 * under the board's power limit. Launches n_workgroups workgroups of 4 waves; every wave issues
 * 16 * iters back-to-back v_mfma_f32_32x32x16_bf16 (32768 flop each) on register operands
 * loaded once from `operands` (device, 8 fragments x 256 lanes x 16 bytes of bf16: fragments
 * 0..3 feed the A side, 4..7 the B side), so no memory traffic occurs inside the loop. out
 * (device) receives n_workgroups * 256 fp32 checksums. Total work: n_workgroups * 4 * 16 *
 * iters * 32768 flop. 1 <= n_workgroups <= 2^20, 1 <= iters <= 2^30.
 */
tp_status tp_mfma_rate_probe(const void* operands, float* out, int64_t n_workgroups, int64_t iters,
                             void* stream);
/*
 * Measurement aid (not part of the shard computation): the HBM read rate that a decode GEMM's
 * access pattern can reach, without its arithmetic. n_workgroups workgroups of 4 waves (two per
 * compute unit, as in the decode GEMMs) each read bytes_per_workgroup contiguous bytes of buf
 * (device; n_workgroups * bytes_per_workgroup bytes) in 8 KB blocks of 16-byte nontemporal loads,
 * the next block in flight while the current one is consumed. out (device) receives
 * n_workgroups * 256 checksums. bytes_per_workgroup a multiple of 8192 in [8192, 2^34];
 * 1 <= n_workgroups <= 2^20; buf 16-byte aligned.
 */
tp_status tp_hbm_read_probe(const void* buf, int64_t bytes_per_workgroup, int64_t n_workgroups, unsigned* out,
                            void* stream);
tp_status tp_profile_read(const char* prefix, double* total_ms, int64_t* launches);
tp_status tp_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
