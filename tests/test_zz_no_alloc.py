"""tp_column_linear_noalloc (the allocation-free variant of tp_column_linear, for callers that
cannot allocate) against tp_column_linear with a workspace, through the C ABI, on two calls in a
row, the second with a smaller input: bitwise equal whenever the call's partial sums fit the
library's 16 MiB static scratch (the few-row regime, and prefill sizes whose tail split fits);
when a prefill split does not fit, its tiles run whole (the same products summed in another
order), and both outputs are held to the bf16 bar against the fp64 oracle."""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from tests._util import assert_close_bf16, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import tensor_transformer_layer_rank_amd as tp
    tp.load()
    return tp


def _arrays(seed, T, K, N):
    rng = np.random.default_rng(seed)
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    return X, W


def _inputs(seed, T, K, N):
    X, W = _arrays(seed, T, K, N)
    return dev(X), dev(W)


def _nan(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


@pytest.mark.parametrize("first,second,out", [
    ((32, 4096, 16000), (8, 1024, 3000), "f32"),      # decode-size LM head, then a smaller one
    ((48, 2048, 6144), (5, 512, 1000), "bf16"),
    ((4100, 1000, 4000), (300, 256, 200), "f32"),     # 272 tiles: 16 split in 4 pieces (16 MiB)
    ((2048, 6464, 5120), (520, 264, 392), "bf16"),    # 160 tiles in 3 pieces: 120 MB, runs whole
])
def test_noalloc_matches_the_workspace_call(tp, first, second, out):
    import torch
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    for i, (T, K, N) in enumerate((first, second)):
        Xh, Wh = _arrays(T + K + N + i, T, K, N)
        X, W = dev(Xh), dev(Wh)
        ref = tp.column_linear(X, W, Y=_nan((T, N), dt))
        got = tp.column_linear_noalloc(X, W, Y=_nan((T, N), dt))
        torch.cuda.synchronize()
        a, b = host(got), host(ref)
        assert np.all(np.isfinite(a)), f"call {i}: unwritten outputs"
        if tp.linear_workspace_size(T, K, N, tp.TP_BF16) <= 16 << 20:
            assert np.array_equal(a, b), f"call {i} ({T}x{K}x{N}): differs from tp_column_linear"
        else:
            exact = O.linear(Xh, Wh)
            assert_close_bf16(a, exact, f"noalloc {T}x{K}x{N} (tiles whole)", out=out)
            assert_close_bf16(b, exact, f"column {T}x{K}x{N} (split)", out=out)


def test_noalloc_refuses_partials_beyond_its_scratch(tp):
    """64 rows x 131072 columns of fp32 partial sums (32 MiB) exceed the 16 MiB scratch."""
    import torch
    X, W = _inputs(1, 64, 512, 131072)
    assert tp.linear_workspace_size(64, 512, 131072, tp.TP_BF16) > 16 << 20
    Y = torch.full((64, 131072), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(tp.TpError) as ei:
        tp.column_linear_noalloc(X, W, Y=Y)
    assert ei.value.name == "TP_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
    assert torch.isnan(Y).all().item(), "a refused call wrote its output"
