"""Plain float64 definitions of a tensor-parallel rank's computation (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the HIP library.

Conventions (the readings of the pages that everything below follows):

* Weights are in X.W orientation, ``W[in, out]``, as in the code example of
  "张量并行：切分 Transformer 层的分布式训练" (实现细节与代码示例) and the worked
  example of "CUDA tensor parallel computations" (最小数学地基).
* Rank ``r`` of ``tp`` owns the r-th contiguous block of columns (column split) or
  of rows (row split); GPU 0 owns the first block in both split examples of
  "CUDA tensor parallel computations" (第二类 Column Parallel, 第三类 Row Parallel).
  Splits must divide evenly (heads are split evenly per "TensorRT LLM 中的并行策略",
  注意力模块).
* Activations are ``[T, H]`` with T = B*S tokens, sequence-major.
* A fused QKV shard holds whole heads: columns [Q_0..Q_{hq-1} | K_0..K_{hkv-1} |
  V_0..V_{hkv-1}], ``d`` contiguous columns per head (each rank keeps whole heads:
  "张量并行：切分 Transformer 层的分布式训练", 自注意力块切分).
* Grouped queries: q head j reads kv head floor(j*hkv/hq).
* Attention is scaled dot-product with scale 1/sqrt(d) (the page names the scaling but
  prints no constant), causal within
  a sequence (key position <= query position), no attention across sequences.
* Rotary embedding (not described on the pages; the rotary base comes with the
  workload): rotate-half pairs (i, i + d/2) with angle pos * theta^(-2i/d), applied
  to Q and K before the scores, position = index within the sequence.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "f64", "column_shard", "row_shard", "linear", "column_linear", "row_linear_partial",
    "all_gather_concat", "partial_sum", "relu", "silu", "apply_act", "mlp_relu_shard",
    "mlp_swiglu_shard", "mlp_shard", "rope_cos_sin", "apply_rope", "softmax_rows",
    "sdpa_causal", "kv_head_of", "split_qkv_heads", "attn_heads", "attn_shard",
    "attn_shard_rows", "attn_shard_weights", "full_attention_block", "decode_qkv",
    "decode_attn_shard", "lm_head_shard", "mlp_full", "rms_norm", "merge_rmsnorm",
    "reduce_scatter_tokens", "linear_backward", "moe_mlp_shard",
]


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Splits ("CUDA tensor parallel computations": 第二类 Column Parallel / 第三类 Row Parallel)
# ---------------------------------------------------------------------------

def column_shard(W, rank: int, tp: int) -> np.ndarray:
    """Columns owned by ``rank``: W[:, rank*N/tp : (rank+1)*N/tp]."""
    W = np.asarray(W)
    N = W.shape[1]
    if N % tp:
        raise ValueError(f"column split: {N} columns do not divide by tp={tp}")
    n = N // tp
    return W[:, rank * n:(rank + 1) * n]


def row_shard(W, rank: int, tp: int) -> np.ndarray:
    """Rows owned by ``rank``: W[rank*K/tp : (rank+1)*K/tp, :]."""
    W = np.asarray(W)
    K = W.shape[0]
    if K % tp:
        raise ValueError(f"row split: {K} rows do not divide by tp={tp}")
    k = K // tp
    return W[rank * k:(rank + 1) * k, :]


def linear(X, W) -> np.ndarray:
    """X @ W in float64 (one output = sum over the shared index of products)."""
    return f64(X) @ f64(W)


# ---------------------------------------------------------------------------
# Element-wise local work ("第五类 局部逐元素计算")
# ---------------------------------------------------------------------------

def relu(z) -> np.ndarray:
    return np.maximum(f64(z), 0.0)


def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    e = np.exp(z[~pos])                       # avoids overflow of exp(-z) for z << 0
    out[~pos] = z[~pos] * e / (1.0 + e)
    return out


def apply_act(z, act: str | None) -> np.ndarray:
    if act in (None, "none"):
        return f64(z)
    if act == "relu":
        return relu(z)
    raise ValueError(f"unknown activation {act!r}")


# ---------------------------------------------------------------------------
# Parallel linear layers
# ---------------------------------------------------------------------------

def column_linear(X, W_shard, act: str | None = None) -> np.ndarray:
    """Column-parallel rank output act(X @ W_shard); X is replicated on every rank."""
    return apply_act(linear(X, W_shard), act)


def row_linear_partial(X_shard, W_shard) -> np.ndarray:
    """Row-parallel rank contribution X_shard @ W_shard (summed across ranks later)."""
    return linear(X_shard, W_shard)


def all_gather_concat(shards) -> np.ndarray:
    """Merge of column-parallel outputs: concatenation along the last axis."""
    return np.concatenate([f64(s) for s in shards], axis=-1)


def partial_sum(partials) -> np.ndarray:
    """Merge of row-parallel outputs: element-wise sum, ((P0 + P1) + P2) + ..."""
    partials = list(partials)
    if not partials:
        raise ValueError("partial_sum needs at least one partial")
    acc = f64(partials[0]).copy()
    for p in partials[1:]:
        acc = acc + f64(p)
    return acc


# ---------------------------------------------------------------------------
# MLP shard ("放进 Transformer": column first, local activation, row second)
# ---------------------------------------------------------------------------

def mlp_relu_shard(X, W1_shard, W2_shard) -> np.ndarray:
    """Rank partial of a ReLU MLP: relu(X @ W1_r) @ W2_r."""
    return linear(relu(linear(X, W1_shard)), W2_shard)


def mlp_swiglu_shard(X, Wg_shard, Wu_shard, Wd_shard) -> np.ndarray:
    """Rank partial of a gated MLP: (SiLU(X @ Wg_r) * (X @ Wu_r)) @ Wd_r."""
    h = silu(linear(X, Wg_shard)) * linear(X, Wu_shard)
    return linear(h, Wd_shard)


def mlp_shard(X, W_gate, W_up, W_down, kind: str) -> np.ndarray:
    if kind == "relu":
        return mlp_relu_shard(X, W_gate, W_down)
    if kind == "swiglu":
        return mlp_swiglu_shard(X, W_gate, W_up, W_down)
    raise ValueError(kind)


def mlp_full(X, W_gate, W_up, W_down, kind: str) -> np.ndarray:
    """Unsharded MLP (the layer a single device would run)."""
    return mlp_shard(X, W_gate, W_up, W_down, kind)


# ---------------------------------------------------------------------------
# Rotary embedding (convention stated in the module docstring; parity unpinned)
# ---------------------------------------------------------------------------

def rope_cos_sin(positions, d: int, theta: float):
    """cos and sin of angle[p, i] = p * theta^(-2i/d), i < d/2; shapes [len(positions), d/2]."""
    if d % 2:
        raise ValueError("rotary embedding needs an even head dimension")
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x, positions, theta: float) -> np.ndarray:
    """Rotate the pairs (x_i, x_{i+d/2}) of each row of x[..., len(positions), d]."""
    x = f64(x)
    d = x.shape[-1]
    cos, sin = rope_cos_sin(positions, d, theta)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


# ---------------------------------------------------------------------------
# Attention for one head ("放进 Transformer": Q_head @ K_head^T, softmax, times V_head)
# ---------------------------------------------------------------------------

def softmax_rows(scores) -> np.ndarray:
    """Row softmax: subtract the row max, exponentiate, normalise (-inf entries give 0)."""
    s = f64(scores)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def sdpa_causal(q, k, v, q_pos=None, k_pos=None) -> np.ndarray:
    """softmax(q k^T / sqrt(d) with -inf where key position > query position) @ v.

    q[Sq, d], k[Sk, d], v[Sk, dv]; positions default to 0..S-1. The whole score
    matrix is formed (the plain definition, not an online/blocked softmax).
    """
    q, k, v = f64(q), f64(k), f64(v)
    d = q.shape[-1]
    q_pos = np.arange(q.shape[0]) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(k.shape[0]) if k_pos is None else np.asarray(k_pos)
    scores = (q @ k.T) / math.sqrt(d)
    scores = np.where(k_pos[None, :] > q_pos[:, None], -np.inf, scores)
    return softmax_rows(scores) @ v


def kv_head_of(j: int, hq: int, hkv: int) -> int:
    """kv head read by q head j when hq query heads share hkv kv heads."""
    if hq % hkv:
        raise ValueError(f"{hq} query heads do not group evenly over {hkv} kv heads")
    return (j * hkv) // hq


def split_qkv_heads(QKV, hq: int, hkv: int, d: int):
    """Split fused projections [T, (hq+2hkv)d] into lists of per-head [T, d] blocks."""
    q = [QKV[:, j * d:(j + 1) * d] for j in range(hq)]
    o = hq * d
    k = [QKV[:, o + g * d:o + (g + 1) * d] for g in range(hkv)]
    o += hkv * d
    v = [QKV[:, o + g * d:o + (g + 1) * d] for g in range(hkv)]
    return q, k, v


def attn_heads(X, W_qkv, B: int, S: int, hq: int, hkv: int, d: int, theta: float) -> np.ndarray:
    """Local attention output [T, hq*d] (heads concatenated) before the O projection."""
    X = f64(X)
    QKV = linear(X, W_qkv)
    q, k, v = split_qkv_heads(QKV, hq, hkv, d)
    out = np.empty((B * S, hq * d), np.float64)
    pos = np.arange(S)
    for b in range(B):
        rows = slice(b * S, (b + 1) * S)
        kr = [apply_rope(k[g][rows], pos, theta) for g in range(hkv)]
        for j in range(hq):
            g = kv_head_of(j, hq, hkv)
            qj = apply_rope(q[j][rows], pos, theta)
            out[rows, j * d:(j + 1) * d] = sdpa_causal(qj, kr[g], v[g][rows])
    return out


def attn_shard(X, W_qkv, W_o, B: int, S: int, hq: int, hkv: int, d: int = 128,
               theta: float = 10000.0) -> np.ndarray:
    """Rank partial of the attention block: concat_j head_j(X) @ W_o[rank rows]."""
    return linear(attn_heads(X, W_qkv, B, S, hq, hkv, d, theta), W_o)


def attn_shard_rows(X, W_qkv, W_o, B: int, S: int, hq: int, hkv: int, d: int,
                    theta: float, rows) -> np.ndarray:
    """The rows ``rows`` (token indices b*S+s) of attn_shard's output, computed alone.

    Row (b, s) depends only on tokens b*S .. b*S+s, so only those are projected.
    """
    X = f64(X)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, W_o.shape[1]), np.float64)
    Wq = f64(W_qkv[:, :hq * d])
    Wk = f64(W_qkv[:, hq * d:(hq + hkv) * d])
    Wv = f64(W_qkv[:, (hq + hkv) * d:])
    Wo = f64(W_o)
    for b in np.unique(rows // S):
        sel = np.nonzero(rows // S == b)[0]
        s_max = int(np.max(rows[sel] % S))
        Xb = X[b * S:b * S + s_max + 1]
        pos = np.arange(s_max + 1)
        K = Xb @ Wk
        V = Xb @ Wv
        kr = [apply_rope(K[:, g * d:(g + 1) * d], pos, theta) for g in range(hkv)]
        for i in sel:
            s = int(rows[i] % S)
            qrow = X[b * S + s:b * S + s + 1] @ Wq
            heads = []
            for j in range(hq):
                g = kv_head_of(j, hq, hkv)
                qj = apply_rope(qrow[:, j * d:(j + 1) * d], [s], theta)
                heads.append(sdpa_causal(qj, kr[g][:s + 1], V[:s + 1, g * d:(g + 1) * d],
                                         q_pos=[s], k_pos=pos[:s + 1]))
            out[i] = (np.concatenate(heads, axis=-1) @ Wo)[0]
    return out


def attn_shard_weights(Wq_full, Wk_full, Wv_full, Wo_full, n_heads: int, n_kv: int,
                       d: int, rank: int, tp: int):
    """The fused QKV column shard and O row shard that rank ``rank`` holds.

    Heads are split evenly (whole heads per rank); when the kv heads are fewer than
    the ranks, each rank keeps a copy of the kv head its query heads read.
    """
    if n_heads % tp:
        raise ValueError("heads must split evenly over the ranks")
    hq = n_heads // tp
    q_cols = Wq_full[:, rank * hq * d:(rank + 1) * hq * d]
    if n_kv >= tp:
        if n_kv % tp:
            raise ValueError("kv heads must split evenly over the ranks")
        hkv = n_kv // tp
        g0 = rank * hkv
    else:
        hkv = 1
        g0 = kv_head_of(rank * hq, n_heads, n_kv)
    k_cols = Wk_full[:, g0 * d:(g0 + hkv) * d]
    v_cols = Wv_full[:, g0 * d:(g0 + hkv) * d]
    W_qkv = np.concatenate([q_cols, k_cols, v_cols], axis=1)
    W_o = Wo_full[rank * hq * d:(rank + 1) * hq * d, :]
    return W_qkv, W_o, hq, hkv


def full_attention_block(X, Wq_full, Wk_full, Wv_full, Wo_full, B: int, S: int,
                         n_heads: int, n_kv: int, d: int, theta: float) -> np.ndarray:
    """The unsharded multi-head attention block (what one device without TP computes)."""
    X = f64(X)
    Q, K, V = linear(X, Wq_full), linear(X, Wk_full), linear(X, Wv_full)
    heads = np.empty((B * S, n_heads * d), np.float64)
    pos = np.arange(S)
    for b in range(B):
        r = slice(b * S, (b + 1) * S)
        for j in range(n_heads):
            g = kv_head_of(j, n_heads, n_kv)
            qj = apply_rope(Q[r, j * d:(j + 1) * d], pos, theta)
            kg = apply_rope(K[r, g * d:(g + 1) * d], pos, theta)
            heads[r, j * d:(j + 1) * d] = sdpa_causal(qj, kg, V[r, g * d:(g + 1) * d])
    return heads @ f64(Wo_full)


# ---------------------------------------------------------------------------
# Decode step (one new token per sequence over a KV cache)
# ---------------------------------------------------------------------------

def decode_qkv(X, W_qkv, hq: int, hkv: int, d: int, pos: int, theta: float):
    """Projected and rotated q [B,hq,d], k [B,hkv,d] and v [B,hkv,d] of the new tokens."""
    QKV = linear(X, W_qkv)
    Bn = QKV.shape[0]
    q = QKV[:, :hq * d].reshape(Bn, hq, d)
    k = QKV[:, hq * d:(hq + hkv) * d].reshape(Bn, hkv, d)
    v = QKV[:, (hq + hkv) * d:].reshape(Bn, hkv, d)
    q = apply_rope(q[:, :, None, :], [pos], theta)[:, :, 0, :]
    k = apply_rope(k[:, :, None, :], [pos], theta)[:, :, 0, :]
    return q, k, v


def decode_attn_shard(X, W_qkv, W_o, k_cache, v_cache, cache_len: int, hq: int,
                      hkv: int, d: int = 128, theta: float = 10000.0):
    """One decode step of the attention shard.

    The new token of each sequence sits at position ``cache_len``; its rotated key
    and value are appended at slot ``cache_len`` and it attends to slots
    0..cache_len. Returns (partial [B, H], k_new [B,hkv,d], v_new [B,hkv,d]).
    """
    q, k, v = decode_qkv(X, W_qkv, hq, hkv, d, cache_len, theta)
    Bn = q.shape[0]
    heads = np.empty((Bn, hq * d), np.float64)
    L = cache_len + 1
    for b in range(Bn):
        for j in range(hq):
            g = kv_head_of(j, hq, hkv)
            keys = np.concatenate([f64(k_cache[b, g, :cache_len]), k[b, g][None]], axis=0)
            vals = np.concatenate([f64(v_cache[b, g, :cache_len]), v[b, g][None]], axis=0)
            heads[b, j * d:(j + 1) * d] = sdpa_causal(q[b, j][None], keys, vals,
                                                       q_pos=[cache_len], k_pos=np.arange(L))[0]
    return linear(heads, W_o), k, v


def lm_head_shard(X, W_lm_shard) -> np.ndarray:
    """Vocabulary-parallel output layer: this rank's logits columns X @ W_lm[:, vocab_r]."""
    return linear(X, W_lm_shard)


# ---------------------------------------------------------------------------
# The step after the merge: residual add and RMS normalisation of the block output
# ---------------------------------------------------------------------------

def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """RMS normalisation over the hidden dimension (last axis): x / sqrt(mean(x^2) + eps) * gamma.

    "CUDA tensor parallel computations", 第五类 局部逐元素计算: a norm reads a whole row of
    the hidden dimension, so on a rank it runs on the merged (replicated) output. The
    pages name RMSNorm without its formula; this is its usual definition (mean of squares
    over the row, eps inside the square root, per-column gain gamma)."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * f64(gamma)


def merge_rmsnorm(partials, residual, gamma, eps: float):
    """Residual stream after a row-parallel block and the next block's normalised input.

    r = residual + (((P_0 + P_1) + ...) + P_{k-1}) (the all-reduce result of
    "CUDA tensor parallel computations", 第四类, added to the block input) and
    normed = rms_norm(r, gamma, eps). Returns (r, normed)."""
    r = f64(residual) + partial_sum(partials)
    return r, rms_norm(r, gamma, eps)


def reduce_scatter_tokens(partials, rank: int, tp: int) -> np.ndarray:
    """This rank's share of a reduce-scatter of row-parallel partials over the token axis:
    the r-th contiguous block of T/tp rows of ((P0 + P1) + ...).

    "CUDA tensor parallel computations", 第四类 跨卡通信计算 (3. reduce-scatter: sum the
    contributions, then cut the result and give each rank only the piece it needs next).
    The cut is along tokens in rank order (the sequence-parallel layout; contiguous blocks,
    rank 0 first, as for the weight splits); T must divide evenly."""
    total = partial_sum(partials)
    T = total.shape[0]
    if T % tp:
        raise ValueError(f"{T} tokens do not split evenly over {tp} ranks")
    n = T // tp
    return total[rank * n:(rank + 1) * n]


# ---------------------------------------------------------------------------
# Backward of a rank's linear shard (the training half of the same split rules)
# ---------------------------------------------------------------------------

def linear_backward(X, W_shard, dY_shard):
    """Gradients of one rank's linear shard Y_r = X_r . W_r: (dX, dW) = (dY_r . W_r^T, X_r^T . dY_r).

    "张量并行：切分 Transformer 层的分布式训练", 列切分 / 行切分 and 前向与反向的通信对称: the same two
    products serve both splits. Column shard (X replicated, dY_r = the gradient of the rank's
    output columns): dX is a partial that the ranks sum; dW_r is local. Row shard (X_r the
    rank's input columns, dY replicated): dX is the rank's slice of the input gradient, complete;
    dW_r is local. The pages only name the collectives; the products are the chain rule."""
    dY = f64(dY_shard)
    return dY @ f64(W_shard).T, f64(X).T @ dY


# ---------------------------------------------------------------------------
# Mixture-of-experts MLP on one rank (experts' weights TP-sharded: "TensorRT LLM 中的并行
# 策略", 混合专家 (MoE): TP and hybrid ETP modes)
# ---------------------------------------------------------------------------

def moe_mlp_shard(X, row_token, expert_offsets, W_gate, W_up, W_down, token_rows, gates) -> np.ndarray:
    """This rank's fp32 partial of a top-k MoE MLP over its local experts.

    The router has chosen up to k experts per token and their gates. Dispatched rows are
    grouped by expert: row r (expert e for offsets[e] <= r < offsets[e+1]) holds token
    row_token[r]; each local expert is an MLP shard with its own column/row-split weights
    (W_gate[e], W_up[e] [H, I_shard], W_down[e] [I_shard, H]), so its row outputs are
    partials like the dense shard's. Token t's partial is the gate-weighted sum of the rows
    token_rows[t, :] (-1, or any index outside the dispatched rows, = a slot whose expert is
    not on this rank), slots in order:
    Y[t] = sum_j gates[t, j] * Yrows[token_rows[t, j]]. Summed over the TP group it is the
    layer's MoE output (the weighted sum is linear, so it commutes with the merge)."""
    X = f64(X)
    offs = [int(v) for v in expert_offsets]
    R = offs[-1]
    rows = np.zeros((R, X.shape[1]), np.float64)
    for e in range(len(offs) - 1):
        a, b = offs[e], offs[e + 1]
        if b > a:
            rows[a:b] = mlp_swiglu_shard(X[np.asarray(row_token[a:b], np.int64)], W_gate[e], W_up[e], W_down[e])
    T = X.shape[0]
    Y = np.zeros((T, X.shape[1]), np.float64)
    tr = np.asarray(token_rows, np.int64)
    g = f64(gates)
    for t in range(T):
        for j in range(tr.shape[1]):
            if 0 <= tr[t, j] < R:
                Y[t] = Y[t] + g[t, j] * rows[tr[t, j]]
    return Y
