"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names what it pins. A plausible slip in the oracle (a dropped term, a
wrong sign, index or scale, a transposed operand, an off-by-one causal mask, a wrong
shard slice) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from oracle import brute
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- printed worked example ("CUDA tensor parallel computations", 最小数学地基 and the split sections)

def test_worked_example_full():
    g = _golden("worked_example.json")
    assert np.array_equal(O.linear(g["X"], g["W"]), np.array(g["full"], float))


def test_worked_example_column_split():
    g = _golden("worked_example.json")
    c = g["column"]
    W = np.array(g["W"], float)
    assert np.array_equal(O.column_shard(W, 0, 2), np.array(c["W0"], float))
    assert np.array_equal(O.column_shard(W, 1, 2), np.array(c["W1"], float))
    y0 = O.column_linear(g["X"], O.column_shard(W, 0, 2))
    y1 = O.column_linear(g["X"], O.column_shard(W, 1, 2))
    assert np.array_equal(y0, np.array(c["Y0"], float))
    assert np.array_equal(y1, np.array(c["Y1"], float))
    assert np.array_equal(O.all_gather_concat([y0, y1]), np.array(c["concat"], float))


def test_worked_example_row_split():
    g = _golden("worked_example.json")
    r = g["row"]
    W = np.array(g["W"], float)
    X = np.array(g["X"], float)
    assert np.array_equal(O.row_shard(W, 0, 2), np.array(r["W0"], float))
    assert np.array_equal(O.row_shard(W, 1, 2), np.array(r["W1"], float))
    assert np.array_equal(O.column_shard(X, 0, 2), np.array(r["X0"], float))
    p0 = O.row_linear_partial(O.column_shard(X, 0, 2), O.row_shard(W, 0, 2))
    p1 = O.row_linear_partial(O.column_shard(X, 1, 2), O.row_shard(W, 1, 2))
    assert np.array_equal(p0, np.array(r["Y0"], float))
    assert np.array_equal(p1, np.array(r["Y1"], float))
    assert np.array_equal(O.partial_sum([p0, p1]), np.array(r["sum"], float))


def test_worked_example_collectives():
    g = _golden("worked_example.json")
    ag, ar = g["all_gather"], g["all_reduce"]
    assert O.all_gather_concat([ag["gpu0_in"], ag["gpu1_in"]]).tolist() == ag["out"]
    assert O.partial_sum([ar["gpu0_in"], ar["gpu1_in"]]).tolist() == ar["out"]


def test_worked_example_products_as_printed():
    # each printed output is x0*W[0][j] + x1*W[1][j]; a transposed W gives different numbers
    X, W = [10, 20], [[1, 2, 3, 4], [5, 6, 7, 8]]
    y = O.linear([X], W)[0]
    for j in range(4):
        assert y[j] == X[0] * W[0][j] + X[1] * W[1][j]


# --- brute force on tiny inputs

@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 2), (4, 7, 6)])
def test_linear_matches_triple_loop(shape):
    rng = np.random.default_rng(11)
    n, k, m = shape
    X = rng.standard_normal((n, k))
    W = rng.standard_normal((k, m))
    ref = np.array(brute.matmul(X.tolist(), W.tolist()))
    np.testing.assert_allclose(O.linear(X, W), ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_column_concat_and_row_sum_equal_unsharded_layer(tp):
    rng = np.random.default_rng(tp)
    X = wl.int_matrix(rng, (5, 16))
    W = wl.int_matrix(rng, (16, 24 if tp != 8 else 32))
    full = np.array(brute.matmul(X.astype(int).tolist(), W.astype(int).tolist()), float)
    cols = [O.column_linear(X, O.column_shard(W, r, tp)) for r in range(tp)]
    assert np.array_equal(O.all_gather_concat(cols), full)
    parts = [O.row_linear_partial(O.column_shard(X, r, tp), O.row_shard(W, r, tp)) for r in range(tp)]
    assert np.array_equal(O.partial_sum(parts), full)


def test_split_rejects_uneven():
    with pytest.raises(ValueError):
        O.column_shard(np.zeros((2, 6)), 0, 4)
    with pytest.raises(ValueError):
        O.row_shard(np.zeros((6, 2)), 0, 4)


def test_config0_mlp_exact_against_integer_brute_force():
    inp = wl.mlp_relu_tp2(0)
    Xi = inp.X.astype(int).tolist()
    W1i, W2i = inp.W_gate.astype(int).tolist(), inp.W_down.astype(int).tolist()
    exact = brute.mlp(Xi, W1i, None, W2i, "relu")           # Python ints: exact
    parts = []
    for r in range(2):
        W1r = O.column_shard(inp.W_gate, r, 2)
        W2r = O.row_shard(inp.W_down, r, 2)
        parts.append(O.mlp_relu_shard(inp.X, W1r, W2r))
    total = O.partial_sum(parts)
    assert np.array_equal(total, np.array(exact, float))
    # every fp32 partial sum along the way is an integer below 2**24, so any order is exact
    assert np.max(np.abs(O.linear(inp.X, inp.W_gate))) <= 64 * 16
    assert max(np.max(np.abs(p)) for p in parts) < 2 ** 24
    assert np.max(np.abs(total)) < 2 ** 24


def test_relu_commutes_with_column_split():
    rng = np.random.default_rng(5)
    X = wl.int_matrix(rng, (6, 8))
    W1 = wl.int_matrix(rng, (8, 16))
    W2 = wl.int_matrix(rng, (16, 8))
    full = O.mlp_full(X, W1, None, W2, "relu")
    for tp in (1, 2, 4, 8):
        parts = [O.mlp_relu_shard(X, O.column_shard(W1, r, tp), O.row_shard(W2, r, tp)) for r in range(tp)]
        assert np.array_equal(O.partial_sum(parts), full)


def test_swiglu_split_invariant():
    inp = wl.random_mlp(7, 9, 16, 32)
    full = O.mlp_full(inp.X, inp.W_gate, inp.W_up, inp.W_down, "swiglu")
    for tp in (2, 4, 8):
        parts = [O.mlp_swiglu_shard(inp.X, O.column_shard(inp.W_gate, r, tp),
                                    O.column_shard(inp.W_up, r, tp), O.row_shard(inp.W_down, r, tp))
                 for r in range(tp)]
        np.testing.assert_allclose(O.partial_sum(parts), full, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kind", ["relu", "swiglu"])
def test_mlp_matches_brute_force(kind):
    inp = wl.random_mlp(3, 4, 6, 10)
    args = [inp.X.tolist(), inp.W_gate.tolist(), inp.W_up.tolist(), inp.W_down.tolist()]
    ref = np.array(brute.mlp(*args, kind))
    got = O.mlp_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down, kind)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_silu_closed_forms():
    assert O.silu([0.0])[0] == 0.0
    np.testing.assert_allclose(O.silu([1.0])[0], 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, rtol=0, atol=1e-12)  # z*s(z) + z*s(-z) = z
    np.testing.assert_allclose(O.silu([50.0, -50.0]), [50.0, -50.0 * math.exp(-50.0)], rtol=1e-12)
    # the activation acts on the gate branch only: swapping gate and up changes the result
    inp = wl.random_mlp(8, 3, 4, 6)
    a = O.mlp_swiglu_shard(inp.X, inp.W_gate, inp.W_up, inp.W_down)
    b = O.mlp_swiglu_shard(inp.X, inp.W_up, inp.W_gate, inp.W_down)
    assert not np.allclose(a, b)


# --- rotary embedding: closed forms (the convention itself is parity unpinned)

def test_rope_position_zero_is_identity_and_norm_preserved():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 16))
    np.testing.assert_array_equal(O.apply_rope(x[:1], [0], 1e4), x[:1])
    y = O.apply_rope(x, np.arange(7) * 37, 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_two_dims_is_rotation_by_position():
    for p in (0, 1, 3, 1024):
        y = O.apply_rope(np.array([[1.0, 0.0]]), [p], 10000.0)[0]
        np.testing.assert_allclose(y, [math.cos(p), math.sin(p)], atol=1e-12)


def test_rope_frequencies_per_pair():
    # d=4: pair (0,2) turns by p, pair (1,3) by p * theta**(-1/2)
    theta, p = 10000.0, 5
    y = O.apply_rope(np.array([[0.0, 1.0, 0.0, 0.0]]), [p], theta)[0]
    a = p * theta ** -0.5
    np.testing.assert_allclose(y, [0.0, math.cos(a), 0.0, math.sin(a)], atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    def dot(m, n):
        return float((O.apply_rope(q, [m], 1e4) @ O.apply_rope(k, [n], 1e4).T)[0, 0])
    assert abs(dot(5, 2) - dot(105, 102)) < 1e-11
    assert abs(dot(7, 7) - float((q @ k.T)[0, 0])) < 1e-11


def test_rope_matches_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 8))
    pos = [0, 4, 999]
    ref = np.array([brute.rope_row(x[i].tolist(), pos[i], 1e4) for i in range(3)])
    np.testing.assert_allclose(O.apply_rope(x, pos, 1e4), ref, rtol=1e-12, atol=1e-12)


# --- scaled dot-product attention

def test_sdpa_single_position_returns_value():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 1, 8))
    np.testing.assert_allclose(O.sdpa_causal(q, k, v), v, rtol=1e-14)


def test_sdpa_first_row_sees_only_first_key():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((3, 5, 8))
    np.testing.assert_allclose(O.sdpa_causal(q, k, v)[0], v[0], rtol=1e-14)


def test_sdpa_equal_keys_give_prefix_mean():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 4))
    k = np.tile(rng.standard_normal((1, 4)), (6, 1))
    v = rng.standard_normal((6, 3))
    out = O.sdpa_causal(q, k, v)
    ref = np.cumsum(v, axis=0) / np.arange(1, 7)[:, None]
    np.testing.assert_allclose(out, ref, rtol=1e-13)


def test_sdpa_scale_is_inverse_sqrt_dim():
    # two keys; score difference = a*2/sqrt(4) = a, so the weights are sigmoid(-a), sigmoid(a)
    a = 0.7
    q = np.array([[0.0, 0.0, 0.0, 0.0], [a, 0.0, 0.0, 0.0]])
    k = np.array([[0.0, 0.0, 0.0, 0.0], [2.0, 0.0, 0.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    out = O.sdpa_causal(q, k, v)[1]
    s = 1.0 / (1.0 + math.exp(-a))
    np.testing.assert_allclose(out, [1.0 - s, s], rtol=1e-14)


def test_sdpa_matches_brute_force_and_rows_are_convex():
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((2, 5, 6))
    v = rng.standard_normal((5, 3))
    ref = np.array(brute.attention_head(q.tolist(), k.tolist(), v.tolist()))
    np.testing.assert_allclose(O.sdpa_causal(q, k, v), ref, rtol=1e-12, atol=1e-13)
    p = O.softmax_rows(np.array([[1.0, 2.0, -np.inf], [0.5, 0.5, 0.5]]))
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-15)
    assert p[0, 2] == 0.0


# --- attention shard: sharding invariants, GQA, sampling, decode

def _mha_full_weights(rng, H, n_heads, n_kv, d):
    def n(shape):
        return rng.standard_normal(shape) * 0.3
    return n((H, n_heads * d)), n((H, n_kv * d)), n((H, n_kv * d)), n((n_heads * d, H))


@pytest.mark.parametrize("n_heads,n_kv,tp", [(4, 4, 1), (4, 4, 2), (4, 4, 4), (8, 2, 2), (8, 2, 4), (4, 1, 4)])
def test_attn_shards_sum_to_full_block(n_heads, n_kv, tp):
    rng = np.random.default_rng(n_heads * 10 + n_kv + tp)
    B, S, H, d = 2, 5, 12, 4
    X = rng.standard_normal((B * S, H))
    Wq, Wk, Wv, Wo = _mha_full_weights(rng, H, n_heads, n_kv, d)
    full = O.full_attention_block(X, Wq, Wk, Wv, Wo, B, S, n_heads, n_kv, d, 100.0)
    parts = []
    for r in range(tp):
        Wqkv, Wo_r, hq, hkv = O.attn_shard_weights(Wq, Wk, Wv, Wo, n_heads, n_kv, d, r, tp)
        parts.append(O.attn_shard(X, Wqkv, Wo_r, B, S, hq, hkv, d, 100.0))
    np.testing.assert_allclose(O.partial_sum(parts), full, rtol=1e-11, atol=1e-12)


def test_attention_block_matches_brute_force():
    rng = np.random.default_rng(21)
    B, S, H, d, nh = 1, 4, 6, 4, 2
    X = rng.standard_normal((B * S, H))
    Wq, Wk, Wv, Wo = _mha_full_weights(rng, H, nh, nh, d)
    Q, K, V = (np.array(brute.matmul(X.tolist(), W.tolist())) for W in (Wq, Wk, Wv))
    heads = []
    for j in range(nh):
        q = [brute.rope_row(Q[t, j * d:(j + 1) * d].tolist(), t, 50.0) for t in range(S)]
        k = [brute.rope_row(K[t, j * d:(j + 1) * d].tolist(), t, 50.0) for t in range(S)]
        heads.append(np.array(brute.attention_head(q, k, V[:, j * d:(j + 1) * d].tolist())))
    ref = np.array(brute.matmul(np.concatenate(heads, axis=1).tolist(), Wo.tolist()))
    got = O.full_attention_block(X, Wq, Wk, Wv, Wo, B, S, nh, nh, d, 50.0)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_gqa_equals_mha_with_copied_kv_head():
    rng = np.random.default_rng(8)
    B, S, H, d, hq = 2, 6, 10, 4, 4
    X = rng.standard_normal((B * S, H))
    Wqkv = rng.standard_normal((H, (hq + 2) * d)) * 0.3
    Wo = rng.standard_normal((hq * d, H))
    gqa = O.attn_shard(X, Wqkv, Wo, B, S, hq, 1, d, 1e4)
    Wq = Wqkv[:, :hq * d]
    Wk = np.tile(Wqkv[:, hq * d:(hq + 1) * d], (1, hq))
    Wv = np.tile(Wqkv[:, (hq + 1) * d:], (1, hq))
    mha = O.attn_shard(X, np.concatenate([Wq, Wk, Wv], 1), Wo, B, S, hq, hq, d, 1e4)
    np.testing.assert_allclose(gqa, mha, rtol=1e-12, atol=1e-13)


def test_heads_are_independent():
    rng = np.random.default_rng(9)
    B, S, H, d, hq = 1, 5, 8, 4, 3
    X = rng.standard_normal((B * S, H))
    Wqkv = rng.standard_normal((H, 3 * hq * d))
    a = O.attn_heads(X, Wqkv, B, S, hq, hq, d, 1e4)
    W2 = Wqkv.copy()
    for base in (0, hq * d, 2 * hq * d):          # perturb head 1's q, k and v columns
        W2[:, base + d:base + 2 * d] += 1.0
    b = O.attn_heads(X, W2, B, S, hq, hq, d, 1e4)
    assert np.array_equal(a[:, :d], b[:, :d]) and np.array_equal(a[:, 2 * d:], b[:, 2 * d:])
    assert not np.allclose(a[:, d:2 * d], b[:, d:2 * d])


def test_no_attention_across_sequences():
    rng = np.random.default_rng(10)
    B, S, H, d = 2, 4, 8, 4
    X = rng.standard_normal((B * S, H))
    Wqkv = rng.standard_normal((H, 3 * d))
    Wo = rng.standard_normal((d, H))
    a = O.attn_shard(X, Wqkv, Wo, B, S, 1, 1, d, 1e4)
    X2 = X.copy()
    X2[S:] += 5.0                                  # change only the second sequence
    b = O.attn_shard(X2, Wqkv, Wo, B, S, 1, 1, d, 1e4)
    assert np.array_equal(a[:S], b[:S])


def test_sampled_rows_match_full_shard():
    inp = wl.random_attn(12, 2, 7, 16, 4, 2, d=4, theta=100.0)
    full = O.attn_shard(inp.X, inp.W_qkv, inp.W_o, inp.B, inp.S, inp.hq, inp.hkv, inp.d, inp.theta)
    rows = [0, 3, 6, 7, 13]
    got = O.attn_shard_rows(inp.X, inp.W_qkv, inp.W_o, inp.B, inp.S, inp.hq, inp.hkv, inp.d,
                            inp.theta, rows)
    np.testing.assert_allclose(got, full[rows], rtol=1e-12, atol=1e-13)


def test_decode_equals_last_row_of_prefill():
    rng = np.random.default_rng(13)
    Bn, p, H, hq, hkv, d, theta = 3, 6, 16, 4, 2, 8, 1e4
    Xseq = rng.standard_normal((Bn, p + 1, H))
    Wqkv = rng.standard_normal((H, (hq + 2 * hkv) * d)) * 0.3
    Wo = rng.standard_normal((hq * d, H))
    # cache = rotated keys and values of positions 0..p-1 of each sequence
    kc = np.zeros((Bn, hkv, p + 4, d))
    vc = np.zeros_like(kc)
    for b in range(Bn):
        QKV = Xseq[b] @ Wqkv
        for g in range(hkv):
            kk = QKV[:p, (hq + g) * d:(hq + g + 1) * d]
            kc[b, g, :p] = O.apply_rope(kk, np.arange(p), theta)
            vc[b, g, :p] = QKV[:p, (hq + hkv + g) * d:(hq + hkv + g + 1) * d]
    dec, knew, vnew = O.decode_attn_shard(Xseq[:, p], Wqkv, Wo, kc, vc, p, hq, hkv, d, theta)
    pre = O.attn_shard(Xseq.reshape(Bn * (p + 1), H), Wqkv, Wo, Bn, p + 1, hq, hkv, d, theta)
    np.testing.assert_allclose(dec, pre[p::p + 1], rtol=1e-11, atol=1e-12)
    QKVl = Xseq[:, p] @ Wqkv
    np.testing.assert_allclose(vnew.reshape(Bn, -1), QKVl[:, (hq + hkv) * d:], rtol=1e-13)


def test_vocab_parallel_logits_concat():
    rng = np.random.default_rng(14)
    X = wl.int_matrix(rng, (3, 8))
    W = wl.int_matrix(rng, (8, 12))
    parts = [O.lm_head_shard(X, O.column_shard(W, r, 2)) for r in range(2)]
    assert np.array_equal(O.all_gather_concat(parts), O.linear(X, W))


def test_partial_sum_is_left_to_right():
    a = np.array([1e16], dtype=np.float64)
    out = O.partial_sum([a, np.array([1.0]), np.array([-1e16])])
    assert out[0] == 0.0          # (1e16 + 1) + (-1e16) rounds to 0 in fp64; other orders give 1
    with pytest.raises(ValueError):
        O.partial_sum([])


# --- input generators (not the method, but both sides rely on them)

def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-5], np.float32)
    y = wl.bf16_round(x)
    assert y[0] == 1.0
    assert y[1] == 1.0                  # halfway: ties to even (mantissa 0)
    assert y[2] == 1.0 + 2 ** -6        # halfway above odd: rounds up to even
    assert y[3] == 1.0
    assert y[4] == -2.5
    assert abs(y[5] - 3.0e-5) <= 3.0e-5 * 2 ** -8
    assert np.array_equal(wl.bf16_round(y), y)


def test_workload_shapes():
    m = wl.mlp_relu_tp2(0)
    assert m.X.shape == (16, 64) and m.W_gate.shape == (64, 256) and m.W_down.shape == (256, 64)
    assert set(np.unique(m.X)).issubset(set(range(-4, 5)))


def test_softmax_is_shift_invariant_at_large_scores():
    p = O.softmax_rows(np.array([[1000.0, 1001.0]]))
    s = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(p[0], [1.0 - s, s], rtol=1e-14)


# ---------------------------------------------------------------- fp8 (OCP E4M3) operands

def test_e4m3_table_matches_library_and_brute_force():
    """All 256 codes: the oracle's table equals torch's float8_e4m3fn decoding and the
    bit-by-bit construction (NaN exactly at 0x7F and 0xFF)."""
    import torch
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = O.e4m3_table()
    bf = np.array([brute.e4m3_to_float(c) for c in range(256)])
    assert np.array_equal(np.isnan(t), np.isnan(lib)) and np.array_equal(np.isnan(t), np.isnan(bf))
    assert np.flatnonzero(np.isnan(t)).tolist() == [0x7F, 0xFF]
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], lib[ok]) and np.array_equal(t[ok], bf[ok])


def test_e4m3_closed_forms():
    t = O.e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x08] == 2.0 ** -6                            # smallest normal
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9   # subnormals
    assert t[0x38] == 1.0 and t[0xC0] == -2.0 and t[0x00] == 0.0
    assert np.signbit(t[0x80]) and t[0x80] == 0.0
    assert np.all(np.diff(t[:0x7F]) > 0)                   # positive codes are ordered


def test_e4m3_quantize_matches_library_in_range():
    """Round-to-nearest-even against torch's conversion, over values inside +-448."""
    import torch
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-12, 9, 100000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_quantize(x), lib)


def test_e4m3_quantize_ties_saturation_and_specials():
    q = O.e4m3_quantize
    # exact midpoints go to the even mantissa
    assert q([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10]).tolist() == [0x38, 0x3A, 0x00, 0x02]
    assert q([448.0, 449.0, 500.0, 1e30, -1e30]).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert q([float("nan"), -0.0, 0.0]).tolist() == [0x7F, 0x80, 0x00]
    # every finite code round-trips
    t = O.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(q(t[codes]), codes)


def test_e4m3_quantize_is_nearest():
    """|value(q(x)) - x| is no larger than the distance to either neighbouring code."""
    rng = np.random.default_rng(9)
    x = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-14, 0, 20000))
    v = O.e4m3_decode(O.e4m3_quantize(x))
    pos = O.e4m3_table()[:0x7F]
    a = np.abs(x)
    best = np.min(np.abs(pos[None, :] - a[:, None]), axis=1)
    assert np.array_equal(np.abs(np.abs(v) - a), best)
    assert np.array_equal(np.signbit(v), np.signbit(x))


def test_fp8_linear_matches_brute_force():
    rng = np.random.default_rng(10)
    Xc = rng.integers(0, 256, (3, 7)).astype(np.uint8)
    Wc = rng.integers(0, 256, (7, 5)).astype(np.uint8)
    Xc[Xc & 0x7F == 0x7F] = 0x12            # keep NaN codes out
    Wc[Wc & 0x7F == 0x7F] = 0x33
    got = O.fp8_linear(Xc, 0.5, Wc, 0.25)
    ref = brute.fp8_matmul(Xc.tolist(), 0.5, Wc.tolist(), 0.25)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-12)


def test_fp8_integer_codes_are_exact():
    """Small integers are exact E4M3 values, so an fp8 layer on them is an integer product."""
    rng = np.random.default_rng(11)
    X = wl.int_matrix(rng, (9, 16))
    W = wl.int_matrix(rng, (16, 12))
    Xc, Wc = O.e4m3_quantize(X), O.e4m3_quantize(W)
    assert np.array_equal(O.e4m3_decode(Xc), X)
    assert np.array_equal(O.fp8_column_linear(Xc, 1.0, Wc, 1.0, "relu"), np.maximum(X.astype(np.float64) @ W, 0))
    assert np.array_equal(O.fp8_row_linear_partial(Xc, 2.0, Wc, 0.5), X.astype(np.float64) @ W)


def test_fp8_mlp_against_brute_force_and_h_codes():
    inp = wl.random_mlp_fp8(12, 4, 32, 8, h_scale=0.125)
    got = O.fp8_mlp_shard(inp.X, inp.x_scale, inp.W_gate, inp.wg_scale, inp.W_up, inp.wu_scale,
                          inp.W_down, inp.wd_scale, inp.h_scale)
    g = brute.fp8_matmul(inp.X.tolist(), inp.x_scale, inp.W_gate.tolist(), inp.wg_scale)
    u = brute.fp8_matmul(inp.X.tolist(), inp.x_scale, inp.W_up.tolist(), inp.wu_scale)
    h = [[a * b for a, b in zip(rg, ru)] for rg, ru in zip(brute.silu(g), u)]
    # h / h_scale in fp32, then the nearest code by exhaustive search (ties: even code)
    finite = [(c, brute.e4m3_to_float(c)) for c in range(256) if not math.isnan(brute.e4m3_to_float(c))]
    hc = []
    for row in h:
        out = []
        for v in row:
            q = float(np.float32(np.float32(v) / np.float32(inp.h_scale)))
            q = max(-448.0, min(448.0, q))
            best = min(finite, key=lambda cv: (abs(cv[1] - q), cv[0] & 1, cv[0] if q >= 0 else -cv[0]))
            out.append(best[0])
        hc.append(out)
    ref = brute.fp8_matmul(hc, inp.h_scale, inp.W_down.tolist(), inp.wd_scale)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-12, atol=1e-12)
    # relu form: h = relu(X W1)
    got_r = O.fp8_mlp_shard(inp.X, inp.x_scale, inp.W_gate, inp.wg_scale, None, 1.0,
                            inp.W_down, inp.wd_scale, inp.h_scale, kind="relu")
    hr = O.fp8_quantize_h(np.maximum(np.array(g), 0), inp.h_scale)
    np.testing.assert_allclose(got_r, O.fp8_linear(hr, inp.h_scale, inp.W_down, inp.wd_scale), rtol=1e-12)


def test_fp8_workload_codes_and_scales():
    inp = wl.random_mlp_fp8(13, 64, 128, 96)
    for codes, scale in ((inp.X, inp.x_scale), (inp.W_gate, inp.wg_scale), (inp.W_down, inp.wd_scale)):
        assert codes.dtype == np.uint8
        v = O.e4m3_decode(codes)
        assert np.all(np.isfinite(v)) and np.max(np.abs(v)) <= 448.0
        assert np.max(np.abs(v)) >= 400.0            # scale = amax / 448 uses the range
        assert scale > 0


# --- residual add + RMSNorm after the merge ("CUDA tensor parallel computations", 第四类 and
# 第五类: a norm needs a whole hidden row, so it follows the all-reduce)

def test_merge_residual_is_input_plus_left_to_right_sum():
    rng = np.random.default_rng(7)
    parts = [rng.integers(-4, 5, size=(3, 8)).astype(np.float32) for _ in range(3)]
    res = rng.integers(-4, 5, size=(3, 8)).astype(np.float32)
    r, _ = O.merge_rmsnorm(parts, res, np.ones(8), 1e-6)
    assert np.array_equal(r, res.astype(float) + parts[0] + parts[1] + parts[2])


def test_rms_norm_worked_numbers():
    # row [3, 4]: mean of squares 12.5; gain [1, 2]
    y = O.rms_norm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(y, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    y = O.rms_norm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.5)   # eps inside the root
    assert np.allclose(y, [[3 / math.sqrt(13.0), 8 / math.sqrt(13.0)]], rtol=0, atol=1e-15)


def test_rms_norm_unit_rms_scale_invariance_and_gain_per_column():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 64))
    y = O.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)         # mean, not sum
    assert np.allclose(O.rms_norm(7.5 * x, np.ones(64), 0.0), y, rtol=1e-13)
    assert np.allclose(O.rms_norm(-x, np.ones(64), 0.0), -y, rtol=1e-13)  # odd in x
    g = rng.standard_normal(64)
    assert np.allclose(O.rms_norm(np.ones((2, 64)), g, 0.0), np.tile(g, (2, 1)), rtol=1e-13)
    assert np.array_equal(O.rms_norm(np.zeros((1, 64)), g, 1e-5), np.zeros((1, 64)))


def test_rms_norm_matches_brute_force():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 24))
    g = rng.standard_normal(24)
    y = O.rms_norm(x, g, 1e-3)
    for i in range(4):
        assert np.allclose(y[i], brute.rms_norm_row(list(x[i]), list(g), 1e-3), rtol=1e-13, atol=0)


def test_reduce_scatter_tokens_concatenates_to_the_sum_and_rejects_uneven():
    rng = np.random.default_rng(10)
    parts = [rng.integers(-4, 5, size=(8, 6)).astype(np.float32) for _ in range(3)]
    pieces = [O.reduce_scatter_tokens(parts, r, 4) for r in range(4)]
    assert all(p.shape == (2, 6) for p in pieces)
    assert np.array_equal(np.concatenate(pieces), parts[0] + parts[1] + parts[2])
    assert np.array_equal(pieces[1], (parts[0] + parts[1] + parts[2])[2:4])   # rank 1: rows 2, 3
    with pytest.raises(ValueError):
        O.reduce_scatter_tokens(parts, 0, 3)


# --- backward of a linear shard (the chain rule of Y = X W; split rules of "张量并行：切分
# Transformer 层的分布式训练", 列切分 / 行切分)

def test_linear_backward_matches_finite_differences():
    rng = np.random.default_rng(11)
    X, W, dY = rng.standard_normal((3, 4)), rng.standard_normal((4, 5)), rng.standard_normal((3, 5))
    dX, dW = O.linear_backward(X, W, dY)
    gX, gW = brute.finite_difference_grads(X.tolist(), W.tolist(), dY.tolist())
    assert np.allclose(dX, gX, rtol=0, atol=1e-8) and np.allclose(dW, gW, rtol=0, atol=1e-8)
    assert dX.shape == X.shape and dW.shape == W.shape


@pytest.mark.parametrize("tp", [2, 4])
def test_linear_backward_split_rules(tp):
    rng = np.random.default_rng(12 + tp)
    X = rng.integers(-3, 4, size=(6, 8)).astype(np.float32)
    W = rng.integers(-3, 4, size=(8, 12)).astype(np.float32)
    dY = rng.integers(-3, 4, size=(6, 12)).astype(np.float32)
    dX_full, dW_full = O.linear_backward(X, W, dY)
    # column shards: dX partials sum to the full dX, dW shards are its column blocks
    cols = [O.linear_backward(X, O.column_shard(W, r, tp), O.column_shard(dY, r, tp)) for r in range(tp)]
    assert np.array_equal(O.partial_sum([c[0] for c in cols]), dX_full)
    assert np.array_equal(np.concatenate([c[1] for c in cols], axis=1), dW_full)
    # row shards: dX shards are the column blocks of dX (complete), dW shards its row blocks
    rows = [O.linear_backward(O.column_shard(X, r, tp), O.row_shard(W, r, tp), dY) for r in range(tp)]
    assert np.array_equal(np.concatenate([r_[0] for r_ in rows], axis=1), dX_full)
    assert np.array_equal(np.concatenate([r_[1] for r_ in rows], axis=0), dW_full)


# --- MoE MLP on one rank ("TensorRT LLM 中的并行策略", 混合专家 (MoE))

def _route(rng, T, E, k):
    """top-k distinct experts per token, gates, and the dispatch grouped by expert."""
    ex = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    gates = rng.random((T, k))
    order = sorted(((int(ex[t, j]), t, j) for t in range(T) for j in range(k)))
    row_token = np.array([t for _, t, _ in order], np.int32)
    offsets = np.searchsorted([e for e, _, _ in order], np.arange(E + 1), side="left")
    token_rows = np.full((T, k), -1, np.int32)
    for r, (_, t, j) in enumerate(order):
        token_rows[t, j] = r
    return row_token, offsets, token_rows, gates


def test_moe_one_expert_identity_routing_is_the_dense_shard():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((6, 8))
    Wg, Wu, Wd = rng.standard_normal((1, 8, 4)), rng.standard_normal((1, 8, 4)), rng.standard_normal((1, 4, 8))
    Y = O.moe_mlp_shard(X, np.arange(6), [0, 6], Wg, Wu, Wd, np.arange(6)[:, None], np.ones((6, 1)))
    assert np.allclose(Y, O.mlp_swiglu_shard(X, Wg[0], Wu[0], Wd[0]), rtol=1e-14, atol=1e-14)


def test_moe_matches_per_token_brute_force_and_is_linear_in_gates():
    rng = np.random.default_rng(14)
    T, H, I, E, k = 5, 6, 4, 3, 2
    X = rng.standard_normal((T, H))
    Wg, Wu, Wd = rng.standard_normal((E, H, I)), rng.standard_normal((E, H, I)), rng.standard_normal((E, I, H))
    row_token, offsets, token_rows, gates = _route(rng, T, E, k)
    token_rows[2, 1] = -1                                   # a slot whose expert is elsewhere
    token_rows[4, 0] = len(row_token) + 3                   # so is a row index past the rows
    Y = O.moe_mlp_shard(X, row_token, offsets, Wg, Wu, Wd, token_rows, gates)
    for t in range(T):
        want = [0.0] * H
        for j in range(k):
            r = token_rows[t, j]
            if r < 0 or r >= len(row_token):
                continue
            e = int(np.searchsorted(offsets, r, side="right") - 1)
            y = brute.mlp([list(X[t])], Wg[e].tolist(), Wu[e].tolist(), Wd[e].tolist(), "swiglu")[0]
            want = [want[i] + gates[t, j] * y[i] for i in range(H)]
        assert np.allclose(Y[t], want, rtol=1e-12, atol=1e-12)
    Y2 = O.moe_mlp_shard(X, row_token, offsets, Wg, Wu, Wd, token_rows, 2.5 * gates)
    assert np.allclose(Y2, 2.5 * Y, rtol=1e-13)


@pytest.mark.parametrize("tp", [2, 4])
def test_moe_tp_within_experts_sums_to_unsharded(tp):
    rng = np.random.default_rng(15 + tp)
    T, H, I, E, k = 7, 8, 16, 4, 2
    X = rng.standard_normal((T, H))
    Wg, Wu, Wd = rng.standard_normal((E, H, I)), rng.standard_normal((E, H, I)), rng.standard_normal((E, I, H))
    route = _route(rng, T, E, k)
    full = O.moe_mlp_shard(X, route[0], route[1], Wg, Wu, Wd, route[2], route[3])
    shards = [O.moe_mlp_shard(X, route[0], route[1],
                              np.stack([O.column_shard(Wg[e], r, tp) for e in range(E)]),
                              np.stack([O.column_shard(Wu[e], r, tp) for e in range(E)]),
                              np.stack([O.row_shard(Wd[e], r, tp) for e in range(E)]), route[2], route[3])
              for r in range(tp)]
    assert np.allclose(O.partial_sum(shards), full, rtol=1e-12, atol=1e-12)
