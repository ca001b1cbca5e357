"""Pure-Python brute force for tiny inputs (test infrastructure only).

These loops restate the definitions element by element with Python floats/ints and
``math`` functions, without NumPy linear algebra, so that the NumPy oracle can be
checked against something other than itself on small cases.
"""
from __future__ import annotations

import math

__all__ = ["matmul", "relu", "silu", "mlp", "attention_head", "rope_row", "e4m3_to_float", "fp8_matmul",
           "rms_norm_row", "finite_difference_grads"]


def matmul(X, W):
    """out[i][j] = sum_k X[i][k] * W[k][j], accumulated left to right."""
    n, kdim, m = len(X), len(W), len(W[0])
    out = []
    for i in range(n):
        row = []
        for j in range(m):
            acc = 0
            for k in range(kdim):
                acc += X[i][k] * W[k][j]
            row.append(acc)
        out.append(row)
    return out


def relu(M):
    return [[x if x > 0 else 0 for x in row] for row in M]


def silu(M):
    return [[x / (1.0 + math.exp(-x)) for x in row] for row in M]


def mlp(X, W_gate, W_up, W_down, kind):
    if kind == "relu":
        return matmul(relu(matmul(X, W_gate)), W_down)
    g, u = silu(matmul(X, W_gate)), matmul(X, W_up)
    h = [[a * b for a, b in zip(rg, ru)] for rg, ru in zip(g, u)]
    return matmul(h, W_down)


def rope_row(x, pos, theta):
    """Rotate pairs (x[i], x[i+d/2]) of one vector by pos * theta**(-2i/d)."""
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        ang = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i + half] * c + x[i] * s
    return out


def attention_head(q, k, v, causal=True):
    """For each query row t: weights over keys u <= t (all keys if not causal)."""
    d = len(q[0])
    out = []
    for t, qt in enumerate(q):
        last = t if causal else len(k) - 1
        scores = []
        for u in range(last + 1):
            s = 0.0
            for c in range(d):
                s += qt[c] * k[u][c]
            scores.append(s / math.sqrt(d))
        m = max(scores)
        w = [math.exp(s - m) for s in scores]
        z = sum(w)
        row = []
        for c in range(len(v[0])):
            acc = 0.0
            for u in range(last + 1):
                acc += w[u] * v[u][c]
            row.append(acc / z)
        out.append(row)
    return out


def e4m3_to_float(code):
    """Value of an OCP E4M3 code, built bit by bit: the 3 mantissa bits are the binary
    fraction after the leading 1 (0 for exponent field 0), scaled by 2^(field - 7)
    (2^-6 for field 0); field 15 with mantissa 7 is NaN."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    field = (code >> 3) & 0xF
    bits = [(code >> 2) & 1, (code >> 1) & 1, code & 1]
    if field == 15 and bits == [1, 1, 1]:
        return float("nan")
    frac = sum(b * 0.5 ** (i + 1) for i, b in enumerate(bits))
    lead = 1.0 if field else 0.0
    power = field - 7 if field else -6
    return sign * (lead + frac) * 2.0 ** power


def fp8_matmul(Xc, x_scale, Wc, w_scale):
    """Element by element: sum_k value(X[i][k]) * value(W[k][j]), times both scales."""
    X = [[e4m3_to_float(c) for c in row] for row in Xc]
    W = [[e4m3_to_float(c) for c in row] for row in Wc]
    return [[v * x_scale * w_scale for v in row] for row in matmul(X, W)]


def rms_norm_row(x, gamma, eps):
    """One row: x_j / sqrt((sum_j x_j^2) / n + eps) * gamma_j, with Python floats."""
    n = len(x)
    ss = 0.0
    for v in x:
        ss += float(v) * float(v)
    inv = 1.0 / math.sqrt(ss / n + float(eps))
    return [float(x[j]) * inv * float(gamma[j]) for j in range(n)]


def finite_difference_grads(X, W, dY, h=1e-3):
    """Central differences of L(X, W) = sum_ij dY_ij (X W)_ij over every entry of X and W."""
    def loss(Xm, Wm):
        P = matmul(Xm, Wm)
        return sum(dY[i][j] * P[i][j] for i in range(len(P)) for j in range(len(P[0])))
    X = [list(map(float, r)) for r in X]
    W = [list(map(float, r)) for r in W]
    gX = [[0.0] * len(X[0]) for _ in X]
    gW = [[0.0] * len(W[0]) for _ in W]
    for M, G in ((X, gX), (W, gW)):
        for i in range(len(M)):
            for j in range(len(M[0])):
                v = M[i][j]
                M[i][j] = v + h
                up = loss(X, W)
                M[i][j] = v - h
                dn = loss(X, W)
                M[i][j] = v
                G[i][j] = (up - dn) / (2 * h)
    return gX, gW
