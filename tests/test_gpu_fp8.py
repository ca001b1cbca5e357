"""GPU parity of the fp8 (OCP E4M3 codes, fp32 per-tensor scales) layers against the
fp64 oracle, through the C ABI.

Every output meets the bf16 bar (relF <= 5e-3, max-abs <= 3e-2, plus half an ulp of a
bf16/fp16 output). fp32 outputs are also held element by element to the precision of
the fp8 matrix instruction: products of two E4M3 values are exact, but the instruction
adds its 64 products with about 15 significant bits relative to the sum of their
magnitudes (measured on gfx950: at most 515 * 2^-24 * sum |x w| for one instruction),
so the bound is |got - ref| <= 2^-14 * (|X| |W|) * x_scale * w_scale + 2^-22 |ref|
(the second term: fp32 rounding of the partial sums across instructions and of the
scale product). In the MLP the intermediate h is
re-encoded: a value within fp32 rounding of a code boundary may take the neighbouring
code there, which the bf16 bar absorbs.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from tests._util import assert_close_bf16, dev_codes, host, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import tensor_transformer_layer_rank_amd as tp
    tp.load()
    return tp


def _codes(rng, shape, std):
    a = (rng.standard_normal(shape) * std).astype(np.float32)
    s = float(np.float32(np.max(np.abs(a)) / 448.0))
    return wl.e4m3_codes(a / s), s


def _assert_sum_bound(got, Xc, xs, Wc, ws, ref, what, terms=1):
    """fp32 accumulation bound (see the module docstring); `terms` results added together."""
    absprod = np.abs(O.e4m3_decode(Xc)) @ np.abs(O.e4m3_decode(Wc)) * (xs * ws)
    bound = terms * (2.0 ** -14 * absprod) + 2.0 ** -22 * np.abs(ref) * terms
    err = np.abs(np.asarray(got, np.float64) - ref)
    worst = float(np.max(err - bound))
    assert worst <= 0, f"{what}: error exceeds the fp32 sum bound by {worst:.3e}"


def _nan(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


@pytest.mark.parametrize("T,K,N,out", [(300, 256, 208, "bf16"), (513, 528, 272, "f32"), (64, 1024, 512, "f16"),
                                       (32, 4096, 1024, "f32"), (1, 64, 16, "f32"), (257, 80, 4096, "bf16")])
def test_fp8_column_linear(tp, T, K, N, out):
    import torch
    rng = np.random.default_rng(T * 3 + K)
    Xc, xs = _codes(rng, (T, K), 1.0)
    Wc, ws = _codes(rng, (K, N), 0.02)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[out]
    Y = tp.column_linear(dev_codes(Xc), dev_codes(Wc), Y=_nan((T, N), dt), scales=(xs, ws))
    torch.cuda.synchronize()
    ref = O.fp8_column_linear(Xc, xs, Wc, ws)
    y = host(Y)
    assert_close_bf16(y, ref, f"fp8 column {T}x{K}x{N} -> {out}", out=out)
    if out == "f32":
        _assert_sum_bound(y, Xc, xs, Wc, ws, ref, "fp8 column")


def test_fp8_column_relu_and_ldy(tp):
    import torch
    rng = np.random.default_rng(4)
    T, K, N, tpn = 200, 128, 96, 3
    Xc, xs = _codes(rng, (T, K), 1.0)
    Wc, ws = _codes(rng, (K, N * tpn), 0.05)
    full = _nan((T, N * tpn), torch.float32)
    for r in range(tpn):
        tp.column_linear(dev_codes(Xc), dev_codes(np.ascontiguousarray(O.column_shard(Wc, r, tpn))),
                         Y=full[:, r * N:], ldy=N * tpn, act=tp.TP_ACT_RELU, scales=(xs, ws))
    torch.cuda.synchronize()
    ref = O.fp8_column_linear(Xc, xs, Wc, ws, "relu")
    assert_close_bf16(host(full), ref, "fp8 relu + ldy concat")
    _assert_sum_bound(host(full), Xc, xs, Wc, ws, ref, "fp8 relu + ldy concat")


@pytest.mark.parametrize("T,K,N", [(300, 272, 144), (64, 2048, 4096), (4200, 592, 4096)])
def test_fp8_row_linear_partial(tp, T, K, N):
    """(4200, 592, 4096): 272 tiles, the 16 past the first round split in 4 K pieces, the
    last piece holding the K tail."""
    import torch
    rng = np.random.default_rng(T + 5 * K)
    Xc, xs = _codes(rng, (T, K), 1.0)
    Wc, ws = _codes(rng, (K, N), 0.02)
    if T == 4200:
        assert tp.linear_workspace_size(T, K, N, tp.TP_FP8_E4M3) > 0, "expected a split grid"
    P = tp.row_linear_partial(dev_codes(Xc), dev_codes(Wc), Y=_nan((T, N), torch.float32), scales=(xs, ws))
    torch.cuda.synchronize()
    ref = O.fp8_row_linear_partial(Xc, xs, Wc, ws)
    assert_close_bf16(host(P), ref, f"fp8 row partial {T}x{K}x{N}")
    _assert_sum_bound(host(P), Xc, xs, Wc, ws, ref, "fp8 row partial")
    tp.row_linear_partial(dev_codes(Xc), dev_codes(Wc), Y=P, accumulate=True, scales=(xs, ws))
    torch.cuda.synchronize()
    _assert_sum_bound(host(P), Xc, xs, Wc, ws, 2 * ref, "fp8 row partial accumulate", terms=2)


def test_fp8_row_partials_sum_to_unsharded_layer(tp):
    import torch
    rng = np.random.default_rng(6)
    T, K, N, tpn = 260, 512, 144, 4
    Xc, xs = _codes(rng, (T, K), 1.0)
    Wc, ws = _codes(rng, (K, N), 0.02)
    parts = [tp.row_linear_partial(dev_codes(np.ascontiguousarray(O.column_shard(Xc, r, tpn))),
                                   dev_codes(np.ascontiguousarray(O.row_shard(Wc, r, tpn))), scales=(xs, ws))
             for r in range(tpn)]
    Y = tp.partial_sum(parts)
    torch.cuda.synchronize()
    _assert_sum_bound(host(Y), Xc, xs, Wc, ws, O.fp8_linear(Xc, xs, Wc, ws), "fp8 sum of row partials", terms=2)


def _mlp(tp, inp, kind="swiglu", rows=None):
    import torch
    k = tp.TP_MLP_SWIGLU if kind == "swiglu" else tp.TP_MLP_RELU
    Y = tp.mlp_shard_fp8(dev_codes(inp.X), dev_codes(inp.W_gate),
                         dev_codes(inp.W_up) if kind == "swiglu" else None, dev_codes(inp.W_down),
                         (inp.x_scale, inp.wg_scale, inp.wu_scale, inp.wd_scale, inp.h_scale),
                         Y=_nan((inp.T, inp.H), torch.float32), kind=k)
    torch.cuda.synchronize()
    X = inp.X if rows is None else inp.X[rows]
    ref = O.fp8_mlp_shard(X, inp.x_scale, inp.W_gate, inp.wg_scale, inp.W_up, inp.wu_scale,
                          inp.W_down, inp.wd_scale, inp.h_scale, kind)
    y = host(Y)
    return (y if rows is None else y[rows]), ref, y


@pytest.mark.parametrize("T,H,I", [(300, 256, 208), (520, 512, 272), (32, 512, 144), (4200, 592, 2048)])
@pytest.mark.parametrize("kind", ["swiglu", "relu"])
def test_fp8_mlp(tp, T, H, I, kind):
    inp = wl.random_mlp_fp8(T + H + I, T, H, I)
    got, ref, _ = _mlp(tp, inp, kind)
    assert_close_bf16(got, ref, f"fp8 mlp {kind} {T}x{H}x{I}")


def test_mlp7b_tp4_fp8_full_size_sampled(tp):
    """mlp7b_tp4's shapes on E4M3 codes: X[4096,4096], gate/up [4096,2752], down [2752,4096]."""
    inp = wl.mlp7b_tp4_fp8()
    rows = sample_rows(4096, 40, seed=2)
    got, ref, y = _mlp(tp, inp, "swiglu", rows)
    assert np.all(np.isfinite(y))
    assert_close_bf16(got, ref, "mlp7b_tp4_fp8 sampled rows")
