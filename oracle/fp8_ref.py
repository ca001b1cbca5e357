"""fp8 (OCP E4M3) operands with per-tensor scales: float64 definitions (test oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

The pages fix the tensor-parallel arithmetic (column split, row split, sum of
partials) but say nothing of number formats beyond it. The fp8 variant reads every
operand as an 8-bit code of the OCP "E4M3" format plus one fp32 scale per tensor:

    value(code) * scale,  value = (-1)^s * 2^(e-7) * (1 + m/8)   (e = 1..15)
                                   (-1)^s * 2^-6  * (m/8)        (e = 0, subnormal)

with bit fields s (1 bit), e (4 bits), m (3 bits); code e = 15, m = 7 is NaN and
there are no infinities (largest magnitude 448). A linear layer on such operands is
the ordinary product of the decoded values, times x_scale * w_scale.

In the fp8 MLP the activated intermediate h is itself stored as E4M3 codes with a
static scale h_scale: code = nearest E4M3 value to h / h_scale (ties to the even
code, magnitudes past 448 saturate to 448). The division and the choice of code are
taken in fp32, the precision the GPU kernel holds h in.
"""
from __future__ import annotations

import math

import numpy as np

from .tp_ref import f64, relu, silu

__all__ = [
    "E4M3_MAX", "e4m3_value", "e4m3_table", "e4m3_decode", "e4m3_quantize", "fp8_linear",
    "fp8_column_linear", "fp8_row_linear_partial", "fp8_quantize_h", "fp8_mlp_shard",
]

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The real number an E4M3 code stands for (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        v = math.ldexp(m / 8.0, -6)
    else:
        v = math.ldexp(1.0 + m / 8.0, e - 7)
    return -v if s else v


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """float64 values of all 256 codes, indexed by code."""
    return _TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    """Elementwise value of uint8 codes, float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# positive finite codes 0x00..0x7E have increasing values
_POS = _TABLE[:0x7F]


def e4m3_quantize(x) -> np.ndarray:
    """Nearest E4M3 code to each value of x (compared in float64): ties go to the code
    with an even mantissa, |x| > 448 saturates to +-448, NaN maps to 0x7F."""
    x = f64(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def fp8_linear(Xc, x_scale: float, Wc, w_scale: float) -> np.ndarray:
    """(value(Xc) @ value(Wc)) * x_scale * w_scale in float64."""
    return (e4m3_decode(Xc) @ e4m3_decode(Wc)) * (float(x_scale) * float(w_scale))


def fp8_column_linear(Xc, x_scale, Wc, w_scale, act: str | None = None) -> np.ndarray:
    """Column-parallel rank output on fp8 operands ("CUDA tensor parallel computations",
    第二类 Column Parallel), optional ReLU (第五类 局部逐元素计算)."""
    y = fp8_linear(Xc, x_scale, Wc, w_scale)
    return relu(y) if act == "relu" else y


def fp8_row_linear_partial(Xc, x_scale, Wc, w_scale) -> np.ndarray:
    """Row-parallel rank partial on fp8 operands (第三类 Row Parallel)."""
    return fp8_linear(Xc, x_scale, Wc, w_scale)


def fp8_quantize_h(h, h_scale: float) -> np.ndarray:
    """E4M3 codes of h / h_scale, the division and the rounding decision in fp32."""
    q = np.asarray(h, dtype=np.float32) / np.float32(h_scale)
    return e4m3_quantize(q.astype(np.float64))


def fp8_mlp_shard(Xc, x_scale, Wgc, wg_scale, Wuc, wu_scale, Wdc, wd_scale, h_scale,
                  kind: str = "swiglu") -> np.ndarray:
    """One rank's MLP on fp8 operands ("张量并行：切分 Transformer 层的分布式训练",
    MLP 块切分): h = SiLU(X Wg) * (X Wu) (or relu(X W1)), stored as E4M3 codes with
    scale h_scale, then the fp32 partial (codes(h) . Wd) * h_scale * wd_scale."""
    g = fp8_linear(Xc, x_scale, Wgc, wg_scale)
    if kind == "relu":
        h = relu(g)
    else:
        h = silu(g) * fp8_linear(Xc, x_scale, Wuc, wu_scale)
    hc = fp8_quantize_h(h, h_scale)
    return fp8_linear(hc, h_scale, Wdc, wd_scale)
