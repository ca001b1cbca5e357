"""tp_column_linear_noalloc (the allocation-free variant of tp_column_linear, for callers that
cannot allocate) against tp_column_linear with a workspace, through the C ABI: bitwise equal
on two calls in a row, the second with a smaller input, in the few-row regime (whose partial
sums live in the library's static scratch) and at a prefill size whose tail split uses it."""
import numpy as np
import pytest

import workloads as wl
from tests._util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    import tensor_transformer_layer_rank_amd as tp
    tp.load()
    return tp


def _inputs(seed, T, K, N):
    rng = np.random.default_rng(seed)
    X = wl.bf16_round(rng.standard_normal((T, K)).astype(np.float32))
    W = wl.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    return dev(X), dev(W)


def _nan(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


@pytest.mark.parametrize("first,second,out", [
    ((32, 4096, 16000), (8, 1024, 3000), "f32"),      # decode-size LM head, then a smaller one
    ((48, 2048, 6144), (5, 512, 1000), "bf16"),
    ((4100, 1000, 4000), (300, 256, 200), "f32"),     # 272 tiles: 16 split in 4 pieces (16 MiB)
    ((2048, 6464, 5120), (520, 264, 392), "bf16"),
])
def test_noalloc_matches_the_workspace_call(tp, first, second, out):
    import torch
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    for i, (T, K, N) in enumerate((first, second)):
        X, W = _inputs(T + K + N + i, T, K, N)
        ref = tp.column_linear(X, W, Y=_nan((T, N), dt))
        got = tp.column_linear_noalloc(X, W, Y=_nan((T, N), dt))
        torch.cuda.synchronize()
        a, b = host(got), host(ref)
        assert np.all(np.isfinite(a)), f"call {i}: unwritten outputs"
        assert np.array_equal(a, b), f"call {i} ({T}x{K}x{N}): differs from tp_column_linear"


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
