"""GPU parity of every libtpshard call against the fp64 oracle (through the C ABI).

Bar: bit-exact on integer-valued fp32; relative Frobenius error <= 5e-3 and max-abs
error <= 3e-2 for bf16 inputs with fp32 accumulation. Outputs are pre-filled with NaN so
that an unwritten tile fails.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as wl
from tests._util import assert_close_bf16, dev, host

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tp():
    import tensor_transformer_layer_rank_amd as tp
    tp.load()
    return tp


def _nan(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


# ---------------------------------------------------------------- exact fp32 path

def test_worked_example_on_gpu(tp):
    import torch
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    X = dev(np.array(g["X"], np.float32), "f32")
    W = np.array(g["W"], np.float32)
    full = torch.empty((1, 4), dtype=torch.float32, device="cuda")
    for r in range(2):   # each rank writes its columns of the full buffer (ldy = 4)
        Wr = dev(np.ascontiguousarray(W[:, 2 * r:2 * r + 2]), "f32")
        tp.column_linear(X, Wr, Y=full[:, 2 * r:], ldy=4)
    torch.cuda.synchronize()
    assert host(full).tolist() == g["column"]["concat"]
    parts = []
    for r, key in enumerate(("X0", "X1")):
        Xr = dev(np.array(g["row"][key], np.float32), "f32")
        Wr = dev(np.array(g["row"]["W%d" % r], np.float32), "f32")
        parts.append(tp.row_linear_partial(Xr, Wr))
    torch.cuda.synchronize()
    assert host(parts[0]).tolist() == g["row"]["Y0"]
    assert host(parts[1]).tolist() == g["row"]["Y1"]
    assert host(tp.partial_sum(parts)).tolist() == g["row"]["sum"]


def test_config0_two_ranks_bit_exact(tp):
    import torch
    inp = wl.mlp_relu_tp2(0)
    X = dev(inp.X, "f32")
    parts_gpu, parts_ref = [], []
    for r in range(2):
        W1 = O.column_shard(inp.W_gate, r, 2)
        W2 = O.row_shard(inp.W_down, r, 2)
        H = tp.column_linear(X, dev(W1, "f32"), act=tp.TP_ACT_RELU)
        P = tp.row_linear_partial(H, dev(W2, "f32"))
        parts_gpu.append(P)
        parts_ref.append(O.mlp_relu_shard(inp.X, W1, W2))
        # the same rank partial through the fused MLP call
        P2 = tp.mlp_shard(X, dev(W1, "f32"), None, dev(W2, "f32"), kind=tp.TP_MLP_RELU)
        torch.cuda.synchronize()
        assert np.array_equal(host(P2), parts_ref[-1])
    Y = tp.partial_sum(parts_gpu)
    torch.cuda.synchronize()
    for r in range(2):
        assert np.array_equal(host(parts_gpu[r]), parts_ref[r])
    assert np.array_equal(host(Y), O.partial_sum(parts_ref))


@pytest.mark.parametrize("T,K,N", [(1, 1, 1), (70, 33, 130), (129, 200, 65), (1030, 72, 1032)])
def test_fp32_linear_ragged_exact(tp, T, K, N):
    """Bit-exact on integer inputs: the 16 x 16 tiles of small products and (1030 x 1032: 289
    tiles of 64 x 64) the large-product tiles, ragged in every dimension, K over one 64-deep tile."""
    import torch
    rng = np.random.default_rng(T + K + N)
    X = wl.int_matrix(rng, (T, K))
    W = wl.int_matrix(rng, (K, N))
    Y = tp.column_linear(dev(X, "f32"), dev(W, "f32"))
    P = tp.row_linear_partial(dev(X, "f32"), dev(W, "f32"))
    torch.cuda.synchronize()
    assert np.array_equal(host(Y), O.linear(X, W))
    assert np.array_equal(host(P), O.linear(X, W))


@pytest.mark.parametrize("k,n", [(1, 5), (2, 64), (3, 1027), (8, 4096 * 33 + 3)])
def test_partial_sum_order_and_tails(tp, k, n):
    import torch
    rng = np.random.default_rng(k * n)
    parts = [rng.standard_normal(n).astype(np.float32) for _ in range(k)]
    out = tp.partial_sum([dev(p, "f32") for p in parts])
    torch.cuda.synchronize()
    ref = parts[0].copy()
    for p in parts[1:]:
        ref = ref + p        # fp32, left to right: the order the call documents
    assert np.array_equal(host(out), ref)


def test_partial_sum_accumulate_in_place(tp):
    import torch
    a = dev(np.arange(12, dtype=np.float32), "f32")
    b = dev(np.ones(12, np.float32), "f32")
    tp.partial_sum([a, b], out=a)
    torch.cuda.synchronize()
    assert host(a).tolist() == (np.arange(12) + 1.0).tolist()


# ---------------------------------------------------------------- merge + residual + RMSNorm

def _merge_call(tp, inp, residual=None, residual_out=None):
    import torch
    T, H = inp.T, inp.H
    parts = [dev(p, "f32") for p in inp.partials]
    res = dev(inp.residual) if residual is None else residual
    R = _nan((T, H), torch.bfloat16) if residual_out is None else residual_out
    R, N = tp.merge_rmsnorm(parts, res, dev(inp.gamma), inp.eps, residual_out=R,
                            normed=_nan((T, H), torch.bfloat16))
    torch.cuda.synchronize()
    return R, N


# H covers every chunk count per thread (1, 2, 4, 8 chunks of 8 for 256 threads) and ragged
# ones (H/8 = 125, 257, 1); k from 1 to 16 partials
@pytest.mark.parametrize("T,H,k", [(5, 136, 1), (37, 1000, 3), (3, 8, 2), (2, 16384, 4), (9, 2056, 16),
                                   (4, 6144, 2)])
def test_merge_rmsnorm_small(tp, T, H, k):
    inp = wl.random_merge(T * 31 + H + k, T, H, k)
    R, N = _merge_call(tp, inp)
    r_ref, n_ref = O.merge_rmsnorm(inp.partials, inp.residual, inp.gamma, inp.eps)
    assert_close_bf16(host(R), r_ref, f"residual T{T} H{H} k{k}", out="bf16")
    assert_close_bf16(host(N), n_ref, f"normed T{T} H{H} k{k}", out="bf16")


def test_merge_rmsnorm_in_place_deterministic_and_zero_rows(tp):
    inp = wl.random_merge(77, 6, 4096, 4)
    R1, N1 = _merge_call(tp, inp)
    res = dev(inp.residual)
    R2, N2 = _merge_call(tp, inp, residual=res, residual_out=res)   # residual updated in place
    assert R2.data_ptr() == res.data_ptr()
    assert np.array_equal(host(R1), host(R2)) and np.array_equal(host(N1), host(N2))
    z = wl.random_merge(78, 3, 1024, 2)
    z.partials = [np.zeros_like(p) for p in z.partials]
    z.residual = np.zeros_like(z.residual)
    R, N = _merge_call(tp, z)
    assert not np.any(host(R)) and not np.any(host(N))               # eps > 0: exact zeros, no NaN


@pytest.mark.parametrize("tp_ranks", [2, 4])
def test_merge_on_token_slices_is_the_sequence_parallel_share(tp, tp_ranks):
    """Sequence-parallel layout: each rank reduce-scatters the partials over tokens and
    normalises only its T/tp rows. The merge call on a rank's row slice (pointer offsets into
    the same buffers) gives exactly the rows of the full call and matches the oracle's
    reduce-scatter share."""
    import torch
    inp = wl.random_merge(91, 64, 2048, 4)
    T, H = inp.T, inp.H
    R_full, N_full = _merge_call(tp, inp)
    parts = [dev(p, "f32") for p in inp.partials]
    res, gamma = dev(inp.residual), dev(inp.gamma)
    n = T // tp_ranks
    for r in range(tp_ranks):
        sl = slice(r * n, (r + 1) * n)
        R, N = tp.merge_rmsnorm([p[sl] for p in parts], res[sl], gamma, inp.eps,
                                residual_out=_nan((n, H), torch.bfloat16), normed=_nan((n, H), torch.bfloat16))
        torch.cuda.synchronize()
        assert np.array_equal(host(R), host(R_full)[sl]) and np.array_equal(host(N), host(N_full)[sl])
        share = O.reduce_scatter_tokens(inp.partials, r, tp_ranks)
        r_ref, n_ref = O.merge_rmsnorm([share], inp.residual[sl], inp.gamma, inp.eps)
        assert_close_bf16(host(R), r_ref, f"rank {r} residual", out="bf16")
        assert_close_bf16(host(N), n_ref, f"rank {r} normed", out="bf16")


def test_merge7b_tp4_full_size(tp):
    """The merge step of the 7B TP=4 block at its full size: [8192, 4096], 4 partials (every
    element of both outputs)."""
    inp = wl.merge7b_tp4()
    R, N = _merge_call(tp, inp)
    R2, N2 = _merge_call(tp, inp)
    r, n = host(R), host(N)
    assert np.array_equal(r, host(R2)) and np.array_equal(n, host(N2)), "two launches differ bitwise"
    r_ref, n_ref = O.merge_rmsnorm(inp.partials, inp.residual, inp.gamma, inp.eps)
    assert_close_bf16(r, r_ref, "merge7b_tp4 residual full output", out="bf16")
    assert_close_bf16(n, n_ref, "merge7b_tp4 normed full output", out="bf16")


# ---------------------------------------------------------------- backward of a linear shard

# partial tiles in every dimension, T below one 256-row tile, K and N not multiples of 128
@pytest.mark.parametrize("T,K,N", [(64, 136, 200), (24, 512, 256), (264, 1000, 72), (520, 256, 1032),
                                   (200, 136, 200), (2056, 1000, 2056)])   # N == T: one paired launch
def test_linear_backward_small(tp, T, K, N):
    import torch
    inp = wl.random_backward(T + 3 * K + 7 * N, T, K, N)
    dX, dW = tp.linear_backward(dev(inp.X), dev(inp.W), dev(inp.dY), dX=_nan((T, K), torch.float32),
                                dW=_nan((K, N), torch.float32))
    torch.cuda.synchronize()
    rX, rW = O.linear_backward(inp.X, inp.W, inp.dY)
    assert_close_bf16(host(dX), rX, f"dX T{T} K{K} N{N}")
    assert_close_bf16(host(dW), rW, f"dW T{T} K{K} N{N}")


def test_linear_backward_split_ranks_sum_to_full(tp):
    """Column shards' dX partials, merged with tp_partial_sum, give the unsharded dX; their dW are
    its column blocks; row shards' dX are its column blocks (GPU products, oracle reference)."""
    import torch
    inp = wl.random_backward(501, 128, 256, 512)
    X, W, dY = dev(inp.X), dev(inp.W), dev(inp.dY)
    rX, rW = O.linear_backward(inp.X, inp.W, inp.dY)
    tpn = 2
    parts, dWs = [], []
    for r in range(tpn):
        cols = slice(r * 256, (r + 1) * 256)
        dXr, dWr = tp.linear_backward(X, W[:, cols].contiguous(), dY[:, cols].contiguous())
        parts.append(dXr)
        dWs.append(dWr)
    full = tp.partial_sum(parts)
    torch.cuda.synchronize()
    assert_close_bf16(host(full), rX, "column shards: summed dX")
    assert_close_bf16(np.concatenate([host(d) for d in dWs], axis=1), rW, "column shards: dW blocks")
    for r in range(tpn):
        rows = slice(r * 128, (r + 1) * 128)
        dXr, dWr = tp.linear_backward(X[:, rows].contiguous(), W[rows].contiguous(), dY)
        torch.cuda.synchronize()
        assert_close_bf16(host(dXr), rX[:, rows], f"row shard {r}: dX slice")
        assert_close_bf16(host(dWr), rW[rows], f"row shard {r}: dW rows")


def test_backward7b_tp4_full_size(tp):
    """Backward of the 7B TP=4 MLP down shard at its full size (every element of dX and dW)."""
    inp = wl.backward7b_tp4()
    X, W, dY = dev(inp.X), dev(inp.W), dev(inp.dY)
    dX, dW = tp.linear_backward(X, W, dY)
    dX2, dW2 = tp.linear_backward(X, W, dY)
    gx, gw = host(dX), host(dW)
    assert np.array_equal(gx, host(dX2)) and np.array_equal(gw, host(dW2)), "two launches differ bitwise"
    ref_x, ref_w = O.linear_backward(inp.X, inp.W, inp.dY)
    assert_close_bf16(gx, ref_x, "backward7b_tp4 dX full output")
    assert_close_bf16(gw, ref_w, "backward7b_tp4 dW full output")


# ---------------------------------------------------------------- MoE MLP shard

def _moe_dev(inp):
    import torch
    return dict(X=dev(inp.X), W_gate=dev(inp.W_gate), W_up=dev(inp.W_up), W_down=dev(inp.W_down),
                expert_offsets=inp.expert_offsets,
                row_token=torch.from_numpy(np.ascontiguousarray(inp.row_token)).cuda(),
                token_rows=torch.from_numpy(np.ascontiguousarray(inp.token_rows)).cuda(),
                gates=dev(inp.gates, "f32"))


def _moe_oracle(inp, tokens=None):
    """The oracle on all tokens, or on a token subset with its rows re-dispatched."""
    if tokens is None:
        return O.moe_mlp_shard(inp.X, inp.row_token, inp.expert_offsets, inp.W_gate, inp.W_up, inp.W_down,
                               inp.token_rows, inp.gates)
    E = inp.W_gate.shape[0]
    eoff = inp.expert_offsets
    slots = sorted((int(np.searchsorted(eoff, r, side="right") - 1), i, j)
                   for i, t in enumerate(tokens) for j, r in enumerate(inp.token_rows[t]) if 0 <= r < eoff[-1])
    row_token = np.array([i for _, i, _ in slots], np.int32)
    offsets = np.searchsorted([e for e, _, _ in slots], np.arange(E + 1), side="left")
    token_rows = np.full((len(tokens), inp.token_rows.shape[1]), -1, np.int32)
    for r, (_, i, j) in enumerate(slots):
        token_rows[i, j] = r
    return O.moe_mlp_shard(inp.X[tokens], row_token, offsets, inp.W_gate, inp.W_up, inp.W_down, token_rows,
                           inp.gates[tokens])


@pytest.mark.parametrize("T,H,I,E,k", [(40, 136, 72, 4, 2), (300, 256, 520, 3, 1), (9, 64, 32, 8, 3)])
def test_moe_mlp_small(tp, T, H, I, E, k):
    import torch
    inp = wl.random_moe(T + H + E, T, H, I, E, k)
    inp.token_rows[1, 0] = -1                          # a slot whose expert is not on this rank
    if T > 2:
        inp.token_rows[2, k - 1] = len(inp.row_token) + 5   # an index outside the rows: skipped
    d = _moe_dev(inp)
    Y = tp.moe_mlp_shard(Y=_nan((T, H), torch.float32), **d)
    Y2 = tp.moe_mlp_shard(**d)
    torch.cuda.synchronize()
    y = host(Y)
    assert np.array_equal(y, host(Y2)), "two launches differ bitwise"
    assert_close_bf16(y, _moe_oracle(inp), f"moe T{T} H{H} I{I} E{E} k{k}")


def test_moe_expert_without_rows_and_unrouted_token(tp):
    import torch
    inp = wl.random_moe(5, 12, 64, 32, 3, 1)
    # every token to expert 0 or 2: expert 1 gets no rows; token 3's only slot is elsewhere
    inp = wl.MoEInputs(inp.name, inp.X, inp.W_gate, inp.W_up, inp.W_down,
                       np.array([0, 6, 6, 12], np.int64), np.array(list(range(6)) + list(range(6, 12)), np.int32),
                       np.arange(12, dtype=np.int32)[:, None].copy(), inp.gates[:, :1] * 0 + 1)
    inp.token_rows[3, 0] = -1
    Y = tp.moe_mlp_shard(Y=_nan((12, 64), torch.float32), **_moe_dev(inp))
    torch.cuda.synchronize()
    y = host(Y)
    assert not np.any(y[3]), "a token without a local slot gets a zero partial"
    assert_close_bf16(y, _moe_oracle(inp), "moe with an empty expert")


def test_moe_no_dispatched_rows(tp):
    """No row reaches this rank's experts: every token's partial is exactly zero."""
    import torch
    inp = wl.random_moe(12, 20, 64, 32, 4, 2)
    inp = wl.MoEInputs(inp.name, inp.X, inp.W_gate, inp.W_up, inp.W_down, np.zeros(5, np.int64),
                       np.zeros(0, np.int32), np.full((20, 2), -1, np.int32), inp.gates)
    d = _moe_dev(inp)
    Y = tp.moe_mlp_shard(Y=_nan((20, 64), torch.float32), **d)
    torch.cuda.synchronize()
    y = host(Y)
    assert np.array_equal(y, np.zeros_like(y))
    assert np.array_equal(y, _moe_oracle(inp))


def test_moe_grouped_skewed_many_experts(tp):
    """A skewed load over 37 experts: more than one grouped launch (32 experts each), experts
    of several row tiles with a ragged last one, small and empty experts between them."""
    import torch
    E = 37
    w = np.ones(E)
    w[0], w[5], w[33], w[36] = 60.0, 25.0, 40.0, 12.0
    w[[2, 3, 20, 34]] = 0.0
    inp = wl.random_moe(11, 700, 128, 96, E, 2, expert_p=w / w.sum())
    counts = np.diff(inp.expert_offsets)
    assert counts.max() > 256 and (counts == 0).sum() == 4 and counts[32:].max() > 64
    Y = tp.moe_mlp_shard(Y=_nan((700, 128), torch.float32), **_moe_dev(inp))
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), _moe_oracle(inp), "moe 37 experts, skewed")


def test_moe8x7b_tp4_full_size(tp):
    """Mixtral-8x7B-like MoE MLP at TP=4 within the experts at full size (every token)."""
    inp = wl.moe8x7b_tp4()
    d = _moe_dev(inp)
    y = host(tp.moe_mlp_shard(**d))
    assert_close_bf16(y, _moe_oracle(inp), "moe8x7b_tp4 full output")


# ---------------------------------------------------------------- bf16 linear layers

@pytest.mark.parametrize("T,K,N", [(300, 256, 200), (513, 520, 264), (256, 64, 256), (65, 4096, 384)])
@pytest.mark.parametrize("out", ["bf16", "f32", "f16"])
def test_column_linear_bf16(tp, T, K, N, out):
    import torch
    rng = np.random.default_rng(T * 7 + N)
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[out]
    Y = tp.column_linear(dev(X), dev(W), Y=_nan((T, N), dt))
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), O.linear(X, W), f"column {T}x{K}x{N} -> {out}", out=out)


@pytest.mark.parametrize("T,K,N", [(5, 1032, 200), (17, 3000, 136), (31, 8, 72), (32, 264, 4104), (33, 776, 520)])
def test_few_row_linear_ragged(tp, T, K, N):
    """The weight-streaming kernels (T <= 64) on odd row counts, K off the 32-row step and the
    128-row staging group (K = 8 included) and N off the 128-column strip: column output in bf16
    and fp32, and the row partial with accumulation."""
    import torch
    rng = np.random.default_rng(11 * T + K + N)
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    ref = O.linear(X, W)
    for out, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        Y = tp.column_linear(dev(X), dev(W), Y=_nan((T, N), dt))
        torch.cuda.synchronize()
        assert_close_bf16(host(Y), ref, f"few-row column {T}x{K}x{N} -> {out}", out=out)
    P = tp.row_linear_partial(dev(X), dev(W), Y=_nan((T, N), torch.float32))
    tp.row_linear_partial(dev(X), dev(W), Y=P, accumulate=True)
    torch.cuda.synchronize()
    assert_close_bf16(host(P), 2 * ref, f"few-row row partial {T}x{K}x{N} accumulate")


@pytest.mark.parametrize("T", [1, 17, 64])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_column_linear_relu_few_rows(tp, T, out):
    """ReLU on the few-row (weight-streaming) path with each output type, K off the chunk step and
    N off the 128-column strip."""
    import torch
    rng = np.random.default_rng(T * 3 + len(out))
    X = wl.bf16_round(rng.standard_normal((T, 1000)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((1000, 392)) * 0.05).astype(np.float32))
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[out]
    Y = tp.column_linear(dev(X), dev(W), Y=_nan((T, 392), dt), act=tp.TP_ACT_RELU)
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), O.relu(O.linear(X, W)), f"few-row relu {T} out {out}", out=out)


def test_column_linear_relu_and_ldy(tp):
    import torch
    rng = np.random.default_rng(3)
    T, K, N, tpn = 200, 128, 96, 3
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N * tpn)) * 0.05).astype(np.float32))
    full = _nan((T, N * tpn), torch.float32)
    for r in range(tpn):
        tp.column_linear(dev(X), dev(np.ascontiguousarray(O.column_shard(W, r, tpn))),
                         Y=full[:, r * N:], ldy=N * tpn, act=tp.TP_ACT_RELU)
    torch.cuda.synchronize()
    assert_close_bf16(host(full), O.relu(O.linear(X, W)), "relu + ldy concat")


@pytest.mark.parametrize("T,K,N", [(300, 264, 136), (64, 2048, 4096), (1, 128, 64), (33, 520, 200)])
def test_row_linear_partial_bf16(tp, T, K, N):
    import torch
    rng = np.random.default_rng(T + 11 * K)
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    P = tp.row_linear_partial(dev(X), dev(W), Y=_nan((T, N), torch.float32))
    torch.cuda.synchronize()
    ref = O.linear(X, W)
    assert_close_bf16(host(P), ref, f"row partial {T}x{K}x{N}")
    tp.row_linear_partial(dev(X), dev(W), Y=P, accumulate=True)
    torch.cuda.synchronize()
    assert_close_bf16(host(P), 2 * ref, "row partial accumulate")


def test_row_partials_sum_to_unsharded_layer(tp):
    import torch
    rng = np.random.default_rng(5)
    T, K, N, tpn = 260, 512, 136, 4
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    parts = [tp.row_linear_partial(dev(np.ascontiguousarray(O.column_shard(X, r, tpn))),
                                   dev(np.ascontiguousarray(O.row_shard(W, r, tpn)))) for r in range(tpn)]
    Y = tp.partial_sum(parts)
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), O.linear(X, W), "sum of row partials")


# Tail split on 256 compute units: the tiles after the last full round are cut along K into
# 2, 3 or 4 pieces whose fp32 partials a fix-up pass sums, when the shorter tail outweighs the
# fix-up (272 tiles: 2 pieces at 10 K steps, 4 at 32; 336 tiles: 3 at 96); grids smaller than
# the machine are cut too (32 tiles: 3 pieces at 32 steps, 4 at 64; 160 tiles: 3 at 202).
# Ragged M, N and K so that the last piece holds the K tail; every output element is compared
# with the oracle, and the split launch with a second launch bitwise.
@pytest.mark.parametrize("T,K,N,out", [(4200, 296, 4096, "bf16"), (4100, 1000, 4000, "f32"),
                                       (5376, 3072, 4096, "f32"), (1000, 1024, 2000, "bf16"),
                                       (1000, 2048, 2000, "f32"), (2048, 6464, 5120, "bf16")])
def test_column_linear_tail_split(tp, T, K, N, out):
    import torch
    rng = np.random.default_rng(T + K)
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    assert tp.linear_workspace_size(T, K, N, tp.TP_BF16) > 0, "expected a split grid"
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[out]
    Y = tp.column_linear(dev(X), dev(W), Y=_nan((T, N), dt))
    Y2 = tp.column_linear(dev(X), dev(W), out_dtype=dt)
    torch.cuda.synchronize()
    y = host(Y)
    assert np.array_equal(y, host(Y2)), "split launches differ bitwise"
    assert_close_bf16(y, O.linear(X, W), f"split column {T}x{K}x{N}", out=out)


def test_row_linear_partial_tail_split_accumulate(tp):
    import torch
    rng = np.random.default_rng(77)
    T, K, N = 4100, 1000, 4000
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    P = tp.row_linear_partial(dev(X), dev(W), Y=_nan((T, N), torch.float32))
    tp.row_linear_partial(dev(X), dev(W), Y=P, accumulate=True)
    torch.cuda.synchronize()
    assert_close_bf16(host(P), 2 * O.linear(X, W), "split row partial accumulate")


@pytest.mark.parametrize("T,H,I,kind", [(300, 256, 200, "swiglu"), (520, 512, 264, "relu"), (4200, 296, 2048, "swiglu"),
                                        (65, 1024, 136, "swiglu")])
def test_mlp_fp16_h(tp, T, H, I, kind):
    """bf16 inputs with h stored in fp16 (down projection on fp16 operands, W_down converted)."""
    import torch
    inp = wl.random_mlp(T + 2 * H + I, T, H, I)
    k = tp.TP_MLP_SWIGLU if kind == "swiglu" else tp.TP_MLP_RELU
    Y = tp.mlp_shard(dev(inp.X), dev(inp.W_gate), dev(inp.W_up) if kind == "swiglu" else None, dev(inp.W_down),
                     Y=_nan((T, H), torch.float32), kind=k, h_dtype=tp.TP_F16)
    torch.cuda.synchronize()
    ref = (O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down) if kind == "swiglu"
           else O.mlp_relu_shard(inp.X, inp.W_gate, inp.W_down))
    rf, _ = assert_close_bf16(host(Y), ref, f"mlp fp16 h {kind} {T}x{H}x{I}")
    assert rf < 1e-3, "an fp16 h should leave far less error than a bf16 one"


def _f16(a):
    """float32 values rounded to IEEE half (input preparation for the fp16-operand calls)."""
    return np.asarray(a, np.float32).astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("T,H,I,kind", [(300, 256, 200, "swiglu"), (520, 512, 264, "relu"), (17, 1024, 1000, "swiglu"),
                                         (64, 512, 264, "relu"), (4100, 1024, 2752, "swiglu")])
def test_mlp_fp16_operands(tp, T, H, I, kind):
    """tp_mlp_shard on fp16 X and weights (h in fp16, fp32 accumulation): the prefill tiles (ragged,
    one grid split past the first round) and the few-row weight-streaming kernels."""
    import torch
    rng = np.random.default_rng(T * 5 + H + I)
    X = _f16(rng.standard_normal((T, H)))
    Wg = _f16(rng.standard_normal((H, I)) * 0.02)
    Wu = _f16(rng.standard_normal((H, I)) * 0.02) if kind == "swiglu" else None
    Wd = _f16(rng.standard_normal((I, H)) * 0.02)
    k = tp.TP_MLP_SWIGLU if kind == "swiglu" else tp.TP_MLP_RELU
    Y = tp.mlp_shard(dev(X, "f16"), dev(Wg, "f16"), dev(Wu, "f16") if Wu is not None else None, dev(Wd, "f16"),
                     Y=_nan((T, H), torch.float32), kind=k)
    torch.cuda.synchronize()
    ref = O.mlp_swiglu_shard(X, Wg, Wu, Wd) if kind == "swiglu" else O.mlp_relu_shard(X, Wg, Wd)
    rf, _ = assert_close_bf16(host(Y), ref, f"mlp fp16 operands {kind} {T}x{H}x{I}")
    assert rf < 1e-3, "fp16 operands and h should leave far less error than bf16 ones"


@pytest.mark.parametrize("T,K,N", [(300, 520, 264), (16, 1024, 392), (64, 4096, 512), (4100, 1000, 4000)])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_column_linear_fp16_operands(tp, T, K, N, out):
    """fp16 X and W (fp32 accumulation): the prefill tiles (ragged, and a grid split past the first
    round) and the few-row weight-streaming kernels."""
    import torch
    rng = np.random.default_rng(T + K + N)
    X = _f16(rng.standard_normal((T, K)))
    W = _f16(rng.standard_normal((K, N)) * 0.05)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[out]
    Y = tp.column_linear(dev(X, "f16"), dev(W, "f16"), Y=_nan((T, N), dt))
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), O.linear(X, W), f"fp16 column {T}x{K}x{N} -> {out}", out=out)


@pytest.mark.parametrize("T,K,N", [(513, 1000, 264), (32, 2048, 4096)])
def test_row_linear_partial_fp16_operands(tp, T, K, N):
    import torch
    rng = np.random.default_rng(3 * T + K)
    X = _f16(rng.standard_normal((T, K)))
    W = _f16(rng.standard_normal((K, N)) * 0.02)
    P = tp.row_linear_partial(dev(X, "f16"), dev(W, "f16"), Y=_nan((T, N), torch.float32))
    torch.cuda.synchronize()
    ref = O.linear(X, W)
    assert_close_bf16(host(P), ref, f"fp16 row partial {T}x{K}x{N}")
    tp.row_linear_partial(dev(X, "f16"), dev(W, "f16"), Y=P, accumulate=True)
    torch.cuda.synchronize()
    assert_close_bf16(host(P), 2 * ref, f"fp16 row partial {T}x{K}x{N} accumulate")


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
def test_mlp_tail_split(tp, kind):
    import torch
    T, H, I = 4200, 296, 2048
    inp = wl.random_mlp(41, T, H, I)
    if kind == "swiglu":
        Y = tp.mlp_shard(dev(inp.X), dev(inp.W_gate), dev(inp.W_up), dev(inp.W_down),
                         Y=_nan((T, H), torch.float32))
        ref = O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down)
    else:
        Y = tp.mlp_shard(dev(inp.X), dev(inp.W_gate), None, dev(inp.W_down), kind=tp.TP_MLP_RELU,
                         Y=_nan((T, H), torch.float32))
        ref = O.mlp_relu_shard(inp.X, inp.W_gate, inp.W_down)
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), ref, f"split mlp {kind}")


# ---------------------------------------------------------------- MLP shard

@pytest.mark.parametrize("T,H,I", [(300, 256, 200), (520, 512, 264), (32, 512, 136), (7, 256, 64)])
def test_mlp_swiglu_small(tp, T, H, I):
    import torch
    inp = wl.random_mlp(T + H + I, T, H, I)
    Y = tp.mlp_shard(dev(inp.X), dev(inp.W_gate), dev(inp.W_up), dev(inp.W_down),
                     Y=_nan((T, H), torch.float32))
    torch.cuda.synchronize()
    ref = O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down)
    assert_close_bf16(host(Y), ref, f"mlp {T}x{H}x{I}")


def test_mlp_relu_bf16(tp):
    import torch
    rng = np.random.default_rng(9)
    T, H, I = 280, 256, 192
    X = wl.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    W1 = wl.bf16_round((rng.standard_normal((H, I)) * 0.05).astype(np.float32))
    W2 = wl.bf16_round((rng.standard_normal((I, H)) * 0.05).astype(np.float32))
    Y = tp.mlp_shard(dev(X), dev(W1), None, dev(W2), kind=tp.TP_MLP_RELU)
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), O.mlp_relu_shard(X, W1, W2), "relu mlp bf16")


def test_mlp_shards_sum_to_unsharded_mlp(tp):
    import torch
    inp = wl.random_mlp(17, 200, 256, 512)
    tpn = 4
    parts = []
    for r in range(tpn):
        parts.append(tp.mlp_shard(dev(inp.X), dev(np.ascontiguousarray(O.column_shard(inp.W_gate, r, tpn))),
                                  dev(np.ascontiguousarray(O.column_shard(inp.W_up, r, tpn))),
                                  dev(np.ascontiguousarray(O.row_shard(inp.W_down, r, tpn)))))
    Y = tp.partial_sum(parts)
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), O.mlp_full(inp.X, inp.W_gate, inp.W_up, inp.W_down, "swiglu"), "sum of mlp shards")


def test_mlp7b_tp4_full_size(tp):
    """LLaMA-7B MLP shard at TP=4 (X[4096,4096], gate/up [4096,2752], down [2752,4096]):
    every element of the fp32 partial against the fp64 oracle, and two launches bitwise equal."""
    import torch
    inp = wl.mlp7b_tp4()
    Xd, Wg, Wu, Wd = dev(inp.X), dev(inp.W_gate), dev(inp.W_up), dev(inp.W_down)
    Y = tp.mlp_shard(Xd, Wg, Wu, Wd, Y=_nan((4096, 4096), torch.float32))
    Y2 = tp.mlp_shard(Xd, Wg, Wu, Wd)
    torch.cuda.synchronize()
    y = host(Y)
    assert np.all(np.isfinite(y))
    assert np.array_equal(y, host(Y2)), "two launches differ bitwise"
    del Y2
    ref = O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down)
    assert_close_bf16(y, ref, "mlp7b_tp4 full output")


# ---------------------------------------------------------------- attention shard

@pytest.mark.parametrize("B,S,hq,hkv,H", [(2, 136, 4, 4, 256), (1, 200, 4, 2, 128), (3, 64, 8, 1, 256), (1, 8, 2, 2, 128),
                                         (1, 1000, 4, 1, 128), (2, 520, 2, 2, 128)])
def test_attn_prefill_small(tp, B, S, hq, hkv, H):
    import torch
    inp = wl.random_attn(B * 100 + S, B, S, H, hq, hkv)
    Y = tp.attn_shard(dev(inp.X), dev(inp.W_qkv), dev(inp.W_o), B, S, hq, hkv,
                      Y=_nan((B * S, H), torch.float32))
    torch.cuda.synchronize()
    ref = O.attn_shard(inp.X, inp.W_qkv, inp.W_o, B, S, hq, hkv, 128, inp.theta)
    assert_close_bf16(host(Y), ref, f"attn B{B} S{S} hq{hq} hkv{hkv}")


def test_attn_shards_sum_to_full_block(tp):
    import torch
    rng = np.random.default_rng(23)
    B, S, H, nh, nkv, d, tpn = 2, 72, 256, 4, 2, 128, 2
    X = wl.bf16_round(rng.standard_normal((B * S, H)).astype(np.float32))
    Wq, Wk, Wv = (wl.bf16_round((rng.standard_normal((H, n * d)) * 0.05).astype(np.float32))
                  for n in (nh, nkv, nkv))
    Wo = wl.bf16_round((rng.standard_normal((nh * d, H)) * 0.05).astype(np.float32))
    parts = []
    for r in range(tpn):
        Wqkv, Wo_r, hq, hkv = O.attn_shard_weights(Wq, Wk, Wv, Wo, nh, nkv, d, r, tpn)
        parts.append(tp.attn_shard(dev(X), dev(np.ascontiguousarray(Wqkv)), dev(np.ascontiguousarray(Wo_r)),
                                   B, S, hq, hkv))
    Y = tp.partial_sum(parts)
    torch.cuda.synchronize()
    ref = O.full_attention_block(X, Wq, Wk, Wv, Wo, B, S, nh, nkv, d, 10000.0)
    assert_close_bf16(host(Y), ref, "sum of attention shards")


def _attn_full_size(tp, inp):
    """The whole fp32 partial of an attention shard against the fp64 oracle."""
    import torch
    T = inp.B * inp.S
    Xd = dev(inp.X)
    Y = tp.attn_shard(Xd, dev(inp.W_qkv), dev(inp.W_o), inp.B, inp.S, inp.hq, inp.hkv,
                      Y=_nan((T, inp.H), torch.float32))
    torch.cuda.synchronize()
    y = host(Y)
    del Y
    assert np.all(np.isfinite(y))
    ref = O.attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.B, inp.S, inp.hq, inp.hkv, inp.d, inp.theta)
    assert_close_bf16(y, ref, inp.name + " attention full output")
    return Xd


def test_attn7b_tp4_full_size(tp):
    """LLaMA-7B attention shard at TP=4: B=4, S=2048, 8 local heads, causal, RoPE 1e4."""
    _attn_full_size(tp, wl.attn7b_tp4())


def test_layer70b_tp8_full_size(tp):
    """70B GQA layer shard at TP=8: attention (8 q heads, 1 kv head) and MLP on the same X,
    every element of both fp32 partials."""
    import torch
    inp = wl.layer70b_tp8()
    Xd = _attn_full_size(tp, inp)
    m = inp.mlp
    # h in fp16: with bf16 h this shard's worst element lands at 2.8e-2 of the 3e-2 bar
    Y = tp.mlp_shard(Xd, dev(m.W_gate), dev(m.W_up), dev(m.W_down), Y=_nan((8192, 8192), torch.float32),
                     h_dtype=tp.TP_F16)
    torch.cuda.synchronize()
    y = host(Y)
    del Y
    assert np.all(np.isfinite(y))
    ref = O.mlp_swiglu_shard(m.X, m.W_gate, m.W_up, m.W_down)
    assert_close_bf16(y, ref, "layer70b_tp8 mlp (fp16 h) full output")


# ---------------------------------------------------------------- decode step

def _decode(tp, inp):
    import torch
    kc, vc = dev(inp.k_cache), dev(inp.v_cache)
    Y = tp.attn_shard(dev(inp.X), dev(inp.W_qkv), dev(inp.W_o), inp.B, 1, inp.hq, inp.hkv,
                      inp.theta, k_cache=kc, v_cache=vc, cache_len=inp.cache_len,
                      Y=_nan((inp.B, inp.H), torch.float32))
    torch.cuda.synchronize()
    return host(Y), host(kc), host(vc)


@pytest.mark.parametrize("B,H,hq,hkv,L,cap", [(4, 256, 2, 2, 37, 40), (3, 512, 4, 1, 300, 301), (32, 256, 2, 2, 1, 8),
                                              (2, 256, 4, 2, 0, 4), (5, 256, 8, 2, 1000, 1003)])
def test_decode_attn_small(tp, B, H, hq, hkv, L, cap):
    inp = wl.random_decode(B + L, B, H, hq, hkv, 64, 64, L, cap)
    y, kc, vc = _decode(tp, inp)
    ref, knew, vnew = O.decode_attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.k_cache, inp.v_cache,
                                          inp.cache_len, inp.hq, inp.hkv, inp.d, inp.theta)
    assert_close_bf16(y, ref, "decode attention")
    assert_close_bf16(kc[:, :, L], knew, "appended keys", out="bf16")
    assert_close_bf16(vc[:, :, L], vnew, "appended values", out="bf16")
    assert np.array_equal(kc[:, :, :L], inp.k_cache[:, :, :L]), "cache prefix modified"


def test_decode7b_tp2_full_size(tp):
    """7B decode step at TP=2: 32 sequences, 16 heads, 1024 cached tokens; MLP and LM head."""
    import torch
    inp = wl.decode7b_tp2()
    y, kc, vc = _decode(tp, inp)
    ref, knew, vnew = O.decode_attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.k_cache, inp.v_cache,
                                          inp.cache_len, inp.hq, inp.hkv, inp.d, inp.theta)
    assert_close_bf16(y, ref, "decode attention partial")
    assert_close_bf16(kc[:, :, inp.cache_len], knew, "appended keys", out="bf16")
    Xd = dev(inp.X)
    Ym = tp.mlp_shard(Xd, dev(inp.W_gate), dev(inp.W_up), dev(inp.W_down), Y=_nan((32, 4096), torch.float32))
    logits = tp.column_linear(Xd, dev(inp.W_lm), Y=_nan((32, 16000), torch.float32))
    torch.cuda.synchronize()
    assert_close_bf16(host(Ym), O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down), "decode mlp")
    assert_close_bf16(host(logits), O.lm_head_shard(inp.X, inp.W_lm), "vocab-parallel logits")


def test_decode_matches_prefill_last_row(tp):
    """Decode at position p with the prefill's own keys/values in the cache = prefill row p."""
    import torch
    B, S, H, hq, hkv = 2, 48, 256, 2, 1
    inp = wl.random_attn(31, B, S, H, hq, hkv)
    p = S - 1
    pre = O.attn_shard(inp.X, inp.W_qkv, inp.W_o, B, S, hq, hkv, 128, inp.theta)
    QKV = O.linear(inp.X, inp.W_qkv)
    kc = np.zeros((B, hkv, S, 128), np.float32)
    vc = np.zeros_like(kc)
    for b in range(B):
        for g in range(hkv):
            kk = QKV[b * S:b * S + p, (hq + g) * 128:(hq + g + 1) * 128]
            kc[b, g, :p] = wl.bf16_round(O.apply_rope(kk, np.arange(p), inp.theta).astype(np.float32))
            vc[b, g, :p] = wl.bf16_round(QKV[b * S:b * S + p, (hq + hkv + g) * 128:(hq + hkv + g + 1) * 128]
                                         .astype(np.float32))
    kd, vd = dev(kc), dev(vc)
    Xl = np.ascontiguousarray(inp.X[p::S])
    Y = tp.attn_shard(dev(Xl), dev(inp.W_qkv), dev(inp.W_o), B, 1, hq, hkv, inp.theta,
                      k_cache=kd, v_cache=vd, cache_len=p)
    torch.cuda.synchronize()
    assert_close_bf16(host(Y), pre[p::S], "decode vs prefill last row")


# ---------------------------------------------------------------- repeatability

def test_repeated_launches_bitwise_equal(tp):
    import torch
    inp = wl.random_attn(41, 2, 256, 512, 4, 2, I=264)
    Xd, Wq, Wo = dev(inp.X), dev(inp.W_qkv), dev(inp.W_o)
    a = host(tp.attn_shard(Xd, Wq, Wo, 2, 256, 4, 2))
    b = host(tp.attn_shard(Xd, Wq, Wo, 2, 256, 4, 2))
    m = inp.mlp
    c = host(tp.mlp_shard(Xd, dev(m.W_gate), dev(m.W_up), dev(m.W_down)))
    d = host(tp.mlp_shard(Xd, dev(m.W_gate), dev(m.W_up), dev(m.W_down)))
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(c, d)


def test_error_is_raised_not_launched(tp):
    import torch
    X = dev(np.zeros((4, 12), np.float32))   # K = 12 is not a multiple of 8 on the bf16 path
    W = dev(np.zeros((12, 16), np.float32))
    with pytest.raises(tp.TpError) as ei:
        tp.column_linear(X, W)
    assert ei.value.name == "TP_ERR_MISALIGNED"
    torch.cuda.synchronize()


# ---------------------------------------------------------------- the fused decode step

def _decode_step(tp, inp, with_lm=True, packed=False):
    import torch
    kc, vc = dev(inp.k_cache), dev(inp.v_cache)
    W = (lambda w: tp.pack_strips(dev(w))) if packed else dev
    I, V = inp.W_gate.shape[1], (inp.W_lm.shape[1] if with_lm else 0)
    Ya, Ym, lg = tp.decode_step(dev(inp.X), W(inp.W_qkv), W(inp.W_o), inp.hq, inp.hkv, inp.theta, kc, vc,
                                inp.cache_len, W(inp.W_gate), W(inp.W_up), W(inp.W_down),
                                W(inp.W_lm) if with_lm else None,
                                Y_attn=_nan((inp.B, inp.H), torch.float32), Y_mlp=_nan((inp.B, inp.H), torch.float32),
                                packed=packed, I=I, V=V)
    torch.cuda.synchronize()
    return host(Ya), host(Ym), (host(lg) if with_lm else None), host(kc), host(vc)


def _check_decode_step(tp, inp, what, with_lm=True, packed=False):
    ya, ym, lg, kc, vc = _decode_step(tp, inp, with_lm, packed)
    L = inp.cache_len
    ref, knew, vnew = O.decode_attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.k_cache, inp.v_cache, L, inp.hq, inp.hkv,
                                          inp.d, inp.theta)
    assert_close_bf16(ya, ref, what + ": attention partial")
    assert_close_bf16(ym, O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down), what + ": mlp partial")
    if with_lm:
        assert_close_bf16(lg, O.lm_head_shard(inp.X, inp.W_lm), what + ": logits")
    assert_close_bf16(kc[:, :, L], knew, what + ": appended keys", out="bf16")
    assert_close_bf16(vc[:, :, L], vnew, what + ": appended values", out="bf16")
    assert np.array_equal(kc[:, :, :L], inp.k_cache[:, :, :L]), "cache prefix modified"
    assert np.array_equal(vc[:, :, :L], inp.v_cache[:, :, :L]), "cache prefix modified"


@pytest.mark.parametrize("B,H,hq,hkv,I,V,L,cap", [(4, 256, 2, 2, 136, 1000, 37, 40), (3, 512, 4, 1, 264, 520, 300, 301),
                                                  (32, 256, 2, 2, 64, 128, 1, 8), (1, 1024, 8, 2, 2048, 4000, 0, 4),
                                                  (64, 512, 4, 4, 1000, 2056, 129, 130)])
def test_decode_step_small(tp, B, H, hq, hkv, I, V, L, cap):
    """tp_decode_step: attention (with cache append), MLP and vocabulary-split head in one call."""
    inp = wl.random_decode(B * 7 + L, B, H, hq, hkv, I, V, L, cap)
    _check_decode_step(tp, inp, f"decode step B{B} H{H} hq{hq} hkv{hkv} I{I} V{V} L{L}")


def test_decode_step_without_head(tp):
    inp = wl.random_decode(5, 8, 512, 4, 2, 264, 64, 100, 104)
    _check_decode_step(tp, inp, "decode step, no output layer", with_lm=False)


def test_decode7b_tp2_fused_step_full_size(tp):
    """The 7B TP=2 decode step through tp_decode_step: 32 sequences, 16 heads, 1024 cached tokens,
    I_shard 5504, vocabulary shard 16000; every output element, and two calls bitwise equal."""
    inp = wl.decode7b_tp2()
    _check_decode_step(tp, inp, "decode7b_tp2 fused step")
    a = _decode_step(tp, inp)
    b = _decode_step(tp, inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "two calls differ bitwise"


# ---------------------------------------------------------------- packed strips

@pytest.mark.parametrize("K,N", [(8, 8), (40, 136), (4096, 16000), (264, 1000), (1, 128)])
def test_pack_strips_layout(tp, K, N):
    """tp_pack_strips moves every element, bit for bit, to [strip][k][column in strip], and zeroes
    the columns past N in the last strip."""
    import torch
    W = np.random.default_rng(K * 7 + N).standard_normal((K, N)).astype(np.float32)
    Wd = dev(W)
    P = host(tp.pack_strips(Wd))
    torch.cuda.synchronize()
    ns = (N + 127) // 128
    ref = np.zeros((K, ns * 128), np.float32)
    ref[:, :N] = host(Wd)
    ref = ref.reshape(K, ns, 128).transpose(1, 0, 2)
    assert P.shape == (ns, K, 128)
    assert np.array_equal(P, ref)


@pytest.mark.parametrize("B,H,hq,hkv,I,V,L,cap", [(4, 256, 2, 2, 136, 1000, 37, 40), (3, 512, 4, 1, 264, 520, 300, 301),
                                                  (32, 256, 2, 2, 64, 128, 1, 8), (1, 1024, 8, 2, 2048, 4000, 0, 4),
                                                  (64, 512, 4, 4, 1000, 2056, 129, 130)])
def test_decode_step_packed_small(tp, B, H, hq, hkv, I, V, L, cap):
    """tp_decode_step_packed: the decode step with every weight in 128-column strips (ragged last
    strips, one token, an empty cache, both activation-row paths)."""
    inp = wl.random_decode(B * 11 + L, B, H, hq, hkv, I, V, L, cap)
    _check_decode_step(tp, inp, f"packed decode step B{B} H{H} hq{hq} hkv{hkv} I{I} V{V} L{L}", packed=True)


def test_decode_step_packed_without_head(tp):
    inp = wl.random_decode(6, 8, 512, 4, 2, 264, 64, 100, 104)
    _check_decode_step(tp, inp, "packed decode step, no output layer", with_lm=False, packed=True)


def test_decode7b_tp2_packed_step_full_size(tp):
    """The 7B TP=2 decode step with packed weights: every output element against the oracle, and
    equal bit for bit to the step on the weights in place (same kernels, same sums)."""
    inp = wl.decode7b_tp2()
    _check_decode_step(tp, inp, "decode7b_tp2 packed step", packed=True)
    a = _decode_step(tp, inp, packed=True)
    b = _decode_step(tp, inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "packed and in-place steps differ bitwise"
