// Backward of one rank's linear shard: dX = dY . W^T and dW = X^T . dY ("张量并行：切分
// Transformer 层的分布式训练", 列切分 / 行切分 and 前向与反向的通信对称: the same two products
// serve a column shard, whose dX is a partial the ranks sum, and a row shard, whose dX is the
// rank's complete slice; dW is local in both).
//
// Both products run on the bf16 MFMA GEMM with one operand read in its stored layout: for dX the
// weight W [K, N] is the transposed B operand (its tile, 256 rows of W by one 32-deep K step,
// has the activation tile's shape and is staged like one), for dW the input X [T, K] is the
// transposed A operand (its tile, one K step of T by 256 columns of X, has the weight tile's
// shape and is read with the transposing LDS loads). Nothing is copied or transposed in HBM.
#include "tp_internal.h"

namespace tpk {

size_t linear_backward_ws_bytes(int64_t T, int64_t K, int64_t N) {
    if (N == T) return gemm_bf16_pair_split_bytes(T, K, K, N, N);
    const size_t a = gemm_bf16_split_bytes(T, K, N, 0), b = gemm_bf16_split_bytes(K, N, T, 0);
    return a > b ? a : b;
}

// dX [T, K] = dY [T, N] . W^T and dW [K, N] = X^T . dY [T, N]. When the two products share
// their inner size (N == T) they run as one launch, so the tail split fills the machine across
// both grids (two 176-tile grids on 256 units would each leave 80 idle). dW's tiles come first:
// the tail round (the launch's last tiles, cut into K pieces) then holds dX tiles, whose
// operands stage without the transposing reads, and the step is ~1% shorter than in the
// other order (backward7b_tp4 on one GPU: 189.8 -> 187.5 us).
hipError_t linear_backward(const void* X, const void* W, const void* dY, float* dX, float* dW, int64_t T,
                           int64_t K, int64_t N, void* ws, hipStream_t s) {
    const size_t ws_bytes = linear_backward_ws_bytes(T, K, N);
    if (N == T)
        return gemm_bf16_f32out_pair_tn_nt(X, dY, dW, K, N, K, N, N, dY, W, dX, T, K, N, N, K, N, ws, ws_bytes, s);
    hipError_t e = gemm_bf16_f32out_t(dY, W, dX, T, K, N, N, N, K, 1, ws, ws_bytes, s);
    if (e != hipSuccess) return e;
    return gemm_bf16_f32out_t(X, dY, dW, K, N, T, K, N, N, 0, ws, ws_bytes, s);
}

}  // namespace tpk
