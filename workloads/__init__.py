"""Seeded synthetic inputs for one tensor-parallel rank's shard.

This module is shared by the fp64 CPU oracle and by the HIP path. It holds no
arithmetic of the method: it only draws random numbers, rounds the draws once to
bfloat16 (round-to-nearest-even) where a workload is bf16, and states shapes.

Workloads (LLaMA-shaped; every draw comes from ``numpy.random.default_rng(seed)`` in
the order the fields are listed):

* ``mlp_relu_tp2``  (seed 0): X[16,64], W1[64,256], W2[256,64]; integers drawn
  uniformly from {-4,...,4}, fp32. The page "CUDA tensor parallel computations"
  (section on the MLP: expand with a column split, local activation, shrink with a
  row split, then sum) is run as two ranks in turn.
* ``mlp7b_tp4``     (seed 1): X[4096,4096] ~ N(0,1); Wg, Wu [4096,2752] and
  Wd [2752,4096] ~ N(0, 0.02). bf16.
* ``attn7b_tp4``    (seed 2): B=4, S=2048, H=4096; Wqkv [4096, 3*1024] (8 local heads of
  128), Wo [1024,4096]. bf16.
* ``layer70b_tp8``  (seed 3): B=4, S=2048, H=8192; Wqkv [8192, (8+1+1)*128],
  Wo [1024,8192], Wg, Wu [8192,3584], Wd [3584,8192]. bf16.
* ``decode7b_tp2``  (seed 4): X[32,4096]; Wqkv [4096, 3*2048], Wo [2048,4096],
  Wg, Wu [4096,5504], Wd [5504,4096], Wlm [4096,16000]; K and V caches
  [32,16,1025,128] whose first 1024 positions are N(0,1) (post-rotation keys). bf16.
* ``mlp7b_tp4_fp8`` (seed 5): the shapes and distributions of ``mlp7b_tp4`` stored as
  OCP E4M3 codes: each tensor is drawn in fp32, given the per-tensor scale
  amax / 448 (fp32), and each draw / scale is rounded to the nearest E4M3 value
  (ties to even). The intermediate h of the MLP gets the static scale 1/8.

"N(0, 0.02)" is read as standard deviation 0.02.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits", "bits_to_f32", "MLPInputs", "AttnInputs", "DecodeInputs",
    "mlp_relu_tp2", "mlp7b_tp4", "attn7b_tp4", "layer70b_tp8", "decode7b_tp2",
    "random_mlp", "random_attn", "random_decode", "int_matrix", "WORKLOADS",
    "e4m3_codes", "FP8MLPInputs", "random_mlp_fp8", "mlp7b_tp4_fp8", "MergeInputs", "random_merge",
    "merge7b_tp4", "BackwardInputs", "random_backward", "backward7b_tp4", "MoEInputs", "random_moe",
    "moe8x7b_tp4",
]


# ---------------------------------------------------------------------------
# bf16 rounding of draws (input preparation, not part of the method)
# ---------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even; return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Expand bfloat16 bit patterns (uint16) to the float32 values they encode."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly the bf16 (RNE) roundings of ``x``."""
    return bits_to_f32(bf16_bits(x))


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no
    infinities): nearest value, ties to even, magnitudes past 448 saturated; uint8 codes.

    Input preparation for fp8 workloads: each value is rounded once to the grid of its
    binade (spacing 2^(e-3) for |x| in [2^e, 2^(e+1)), e >= -6; spacing 2^-9 below 2^-6).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)
    r = np.round(a / step) * step            # numpy rounds halves to even
    r = np.minimum(r, 448.0)
    # fields of the rounded magnitude
    with np.errstate(divide="ignore"):
        er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, er + 7, 0)
    man_field = np.where(normal, r / np.exp2(er) * 8 - 8, r * 2.0 ** 9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(man_field).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_round(a)


def int_matrix(rng: np.random.Generator, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integers drawn uniformly from {lo, ..., hi} (inclusive), stored as float32."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


# ---------------------------------------------------------------------------
# Containers
# ---------------------------------------------------------------------------

@dataclass
class MLPInputs:
    name: str
    X: np.ndarray                  # [T, H]
    W_gate: np.ndarray             # [H, I]  (W1 for the ReLU form)
    W_up: np.ndarray | None        # [H, I]  (None for the ReLU form)
    W_down: np.ndarray             # [I, H]  (W2 for the ReLU form)
    kind: str                      # "relu" | "swiglu"
    dtype: str                     # "f32" | "bf16"
    tp: int = 1                    # how many ranks the full weights are split over
    full: bool = False             # True: W_* are the unsharded weights (split by rank)

    @property
    def T(self): return self.X.shape[0]

    @property
    def H(self): return self.X.shape[1]

    @property
    def I(self): return self.W_gate.shape[1]


@dataclass
class AttnInputs:
    name: str
    X: np.ndarray                  # [B*S, H], sequence-major
    W_qkv: np.ndarray              # [H, (hq + 2*hkv) * d]  columns: Q heads | K heads | V heads
    W_o: np.ndarray                # [hq*d, H]
    B: int
    S: int
    hq: int
    hkv: int
    d: int = 128
    theta: float = 10000.0
    mlp: MLPInputs | None = None   # layer shard: MLP on the same X

    @property
    def H(self): return self.X.shape[1]


@dataclass
class DecodeInputs:
    name: str
    X: np.ndarray                  # [B, H]  one new token per sequence
    W_qkv: np.ndarray              # [H, (hq + 2*hkv) * d]
    W_o: np.ndarray                # [hq*d, H]
    W_gate: np.ndarray
    W_up: np.ndarray
    W_down: np.ndarray
    W_lm: np.ndarray               # [H, V_shard]
    k_cache: np.ndarray            # [B, hkv, cap, d]; positions < cache_len hold keys
    v_cache: np.ndarray            # [B, hkv, cap, d]
    cache_len: int
    hq: int
    hkv: int
    d: int = 128
    theta: float = 10000.0

    @property
    def B(self): return self.X.shape[0]

    @property
    def H(self): return self.X.shape[1]


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

def mlp_relu_tp2(seed: int = 0) -> MLPInputs:
    """fp32 TP=2 MLP with integer values; full (unsharded) W1[64,256], W2[256,64]."""
    rng = np.random.default_rng(seed)
    X = int_matrix(rng, (16, 64))
    W1 = int_matrix(rng, (64, 256))
    W2 = int_matrix(rng, (256, 64))
    return MLPInputs("mlp_relu_tp2", X, W1, None, W2, "relu", "f32", tp=2, full=True)


def random_mlp(seed: int, T: int, H: int, I: int, name: str = "mlp") -> MLPInputs:
    rng = np.random.default_rng(seed)
    X = _normal(rng, (T, H), 1.0)
    Wg = _normal(rng, (H, I), 0.02)
    Wu = _normal(rng, (H, I), 0.02)
    Wd = _normal(rng, (I, H), 0.02)
    return MLPInputs(name, X, Wg, Wu, Wd, "swiglu", "bf16")


def mlp7b_tp4(seed: int = 1) -> MLPInputs:
    """LLaMA-7B MLP shard at TP=4: X[4096,4096]; gate/up [4096,2752]; down [2752,4096]."""
    return random_mlp(seed, 4096, 4096, 2752, "mlp7b_tp4")


def random_attn(seed: int, B: int, S: int, H: int, hq: int, hkv: int, d: int = 128,
                theta: float = 10000.0, I: int = 0, name: str = "attn") -> AttnInputs:
    rng = np.random.default_rng(seed)
    X = _normal(rng, (B * S, H), 1.0)
    Wqkv = _normal(rng, (H, (hq + 2 * hkv) * d), 0.02)
    Wo = _normal(rng, (hq * d, H), 0.02)
    mlp = None
    if I:
        Wg = _normal(rng, (H, I), 0.02)
        Wu = _normal(rng, (H, I), 0.02)
        Wd = _normal(rng, (I, H), 0.02)
        mlp = MLPInputs(name + ".mlp", X, Wg, Wu, Wd, "swiglu", "bf16")
    return AttnInputs(name, X, Wqkv, Wo, B, S, hq, hkv, d, theta, mlp)


def attn7b_tp4(seed: int = 2) -> AttnInputs:
    """LLaMA-7B attention shard at TP=4: B=4, S=2048, H=4096, 8 local heads of 128."""
    return random_attn(seed, 4, 2048, 4096, 8, 8, name="attn7b_tp4")


def layer70b_tp8(seed: int = 3) -> AttnInputs:
    """70B GQA layer shard at TP=8: 8 q heads, 1 kv head, H=8192, MLP shard I=3584."""
    return random_attn(seed, 4, 2048, 8192, 8, 1, I=3584, name="layer70b_tp8")


def random_decode(seed: int, B: int, H: int, hq: int, hkv: int, I: int, V: int,
                  cache_len: int, cap: int, d: int = 128, theta: float = 10000.0,
                  name: str = "decode") -> DecodeInputs:
    rng = np.random.default_rng(seed)
    X = _normal(rng, (B, H), 1.0)
    Wqkv = _normal(rng, (H, (hq + 2 * hkv) * d), 0.02)
    Wo = _normal(rng, (hq * d, H), 0.02)
    Wg = _normal(rng, (H, I), 0.02)
    Wu = _normal(rng, (H, I), 0.02)
    Wd = _normal(rng, (I, H), 0.02)
    Wlm = _normal(rng, (H, V), 0.02)
    kc = np.zeros((B, hkv, cap, d), np.float32)
    vc = np.zeros((B, hkv, cap, d), np.float32)
    kc[:, :, :cache_len, :] = _normal(rng, (B, hkv, cache_len, d), 1.0)
    vc[:, :, :cache_len, :] = _normal(rng, (B, hkv, cache_len, d), 1.0)
    return DecodeInputs(name, X, Wqkv, Wo, Wg, Wu, Wd, Wlm, kc, vc, cache_len, hq, hkv, d, theta)


def decode7b_tp2(seed: int = 4) -> DecodeInputs:
    """7B decode step at TP=2: 32 sequences, 16 local heads, 1024 cached tokens, LM head 16000."""
    return random_decode(seed, 32, 4096, 16, 16, 5504, 16000, 1024, 1025, name="decode7b_tp2")


@dataclass
class FP8MLPInputs:
    """An MLP shard whose X and weights are E4M3 codes (uint8) with fp32 per-tensor scales."""
    name: str
    X: np.ndarray                  # [T, H] uint8
    x_scale: float
    W_gate: np.ndarray             # [H, I] uint8
    wg_scale: float
    W_up: np.ndarray               # [H, I] uint8
    wu_scale: float
    W_down: np.ndarray             # [I, H] uint8
    wd_scale: float
    h_scale: float                 # static scale of the intermediate h

    @property
    def T(self): return self.X.shape[0]

    @property
    def H(self): return self.X.shape[1]

    @property
    def I(self): return self.W_gate.shape[1]


def _fp8_tensor(rng: np.random.Generator, shape, std: float):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    scale = np.float32(np.max(np.abs(a)) / np.float32(448.0))
    return e4m3_codes(a / scale), float(scale)


def random_mlp_fp8(seed: int, T: int, H: int, I: int, name: str = "mlp_fp8",
                   h_scale: float = 0.125) -> FP8MLPInputs:
    rng = np.random.default_rng(seed)
    X, xs = _fp8_tensor(rng, (T, H), 1.0)
    Wg, gs = _fp8_tensor(rng, (H, I), 0.02)
    Wu, us = _fp8_tensor(rng, (H, I), 0.02)
    Wd, ds = _fp8_tensor(rng, (I, H), 0.02)
    return FP8MLPInputs(name, X, xs, Wg, gs, Wu, us, Wd, ds, h_scale)


def mlp7b_tp4_fp8(seed: int = 5) -> FP8MLPInputs:
    """mlp7b_tp4's shapes as E4M3 codes: X[4096,4096], gate/up [4096,2752], down [2752,4096]."""
    return random_mlp_fp8(seed, 4096, 4096, 2752, "mlp7b_tp4_fp8")


@dataclass
class MergeInputs:
    """The step after a row-parallel block's merge: k fp32 partials, the bf16 residual stream
    and the bf16 RMSNorm gain."""
    name: str
    partials: list                 # k x [T, H] float32
    residual: np.ndarray           # [T, H] float32, bf16-rounded
    gamma: np.ndarray              # [H] float32, bf16-rounded
    eps: float

    @property
    def T(self): return self.residual.shape[0]

    @property
    def H(self): return self.residual.shape[1]


def random_merge(seed: int, T: int, H: int, k: int, eps: float = 1e-5, name: str = "merge") -> MergeInputs:
    """Partials N(0, 0.5^2) in fp32 (GEMM outputs), residual N(0,1) and gain 1 + N(0, 0.1^2),
    both bf16-rounded."""
    rng = np.random.default_rng(seed)
    partials = [rng.standard_normal(size=(T, H), dtype=np.float32) * np.float32(0.5) for _ in range(k)]
    residual = _normal(rng, (T, H), 1.0)
    gamma = bf16_round(np.float32(1.0) + _normal(rng, (H,), 0.1))
    return MergeInputs(name, partials, residual, gamma, eps)


def merge7b_tp4(seed: int = 6) -> MergeInputs:
    """Merge step of the 7B TP=4 block: the 4 ranks' fp32 partials of [8192, 4096] (B=4,
    S=2048) summed into the residual stream, then RMSNorm (eps 1e-5)."""
    return random_merge(seed, 8192, 4096, 4, 1e-5, name="merge7b_tp4")


@dataclass
class BackwardInputs:
    """Backward of one rank's linear shard: forward input X, weight shard W, output gradient dY."""
    name: str
    X: np.ndarray      # [T, K] float32, bf16-rounded
    W: np.ndarray      # [K, N] float32, bf16-rounded
    dY: np.ndarray     # [T, N] float32, bf16-rounded


def random_backward(seed: int, T: int, K: int, N: int, name: str = "backward") -> BackwardInputs:
    """X N(0,1), W N(0, 0.02^2), dY N(0,1), all bf16-rounded."""
    rng = np.random.default_rng(seed)
    return BackwardInputs(name, _normal(rng, (T, K), 1.0), _normal(rng, (K, N), 0.02), _normal(rng, (T, N), 1.0))


def backward7b_tp4(seed: int = 7) -> BackwardInputs:
    """Backward of the 7B TP=4 MLP down shard (row-parallel): X = h [4096, 2752],
    W_down shard [2752, 4096], dY [4096, 4096] replicated."""
    return random_backward(seed, 4096, 2752, 4096, name="backward7b_tp4")


@dataclass
class MoEInputs:
    """A top-k MoE MLP on one rank: tokens, the local experts' TP-sharded SwiGLU weights and a
    router's choice laid out as the dispatch (rows grouped by expert) and the combine map."""
    name: str
    X: np.ndarray              # [T, H] float32, bf16-rounded
    W_gate: np.ndarray         # [E, H, I] float32, bf16-rounded
    W_up: np.ndarray           # [E, H, I]
    W_down: np.ndarray         # [E, I, H]
    expert_offsets: np.ndarray # [E+1] int64
    row_token: np.ndarray      # [R] int32
    token_rows: np.ndarray     # [T, k] int32
    gates: np.ndarray          # [T, k] float32


def random_moe(seed: int, T: int, H: int, I: int, E: int, k: int, name: str = "moe",
               expert_p=None) -> MoEInputs:
    """X N(0,1), weights N(0, 0.02^2) (bf16-rounded); every token picks k distinct experts
    uniformly at random (or drawn without replacement with probabilities expert_p, for skewed
    loads) with gates uniform in (0, 1) scaled to sum to 1; dispatched rows are ordered by
    (expert, token, slot)."""
    rng = np.random.default_rng(seed)
    X = _normal(rng, (T, H), 1.0)
    Wg, Wu, Wd = _normal(rng, (E, H, I), 0.02), _normal(rng, (E, H, I), 0.02), _normal(rng, (E, I, H), 0.02)
    if expert_p is None:
        experts = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    else:
        experts = np.array([rng.choice(E, size=k, replace=False, p=expert_p) for _ in range(T)]).reshape(T, k)
    g = rng.random((T, k)).astype(np.float32) + np.float32(1e-3)
    gates = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    key = experts.astype(np.int64) * (T * k) + np.arange(T)[:, None] * k + np.arange(k)[None, :]
    order = np.argsort(key.ravel(), kind="stable")
    row_token = (order // k).astype(np.int32)
    counts = np.bincount(experts.ravel(), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    token_rows = np.empty(T * k, np.int32)
    token_rows[order] = np.arange(T * k, dtype=np.int32)
    return MoEInputs(name, X, Wg, Wu, Wd, offsets, row_token, token_rows.reshape(T, k), gates)


def moe8x7b_tp4(seed: int = 8) -> MoEInputs:
    """Mixtral-8x7B-like MoE MLP at TP=4 within the experts: 2048 tokens, H 4096, the 8
    experts' I = 14336 split 4 ways (3584), top-2 routing."""
    return random_moe(seed, 2048, 4096, 3584, 8, 2, name="moe8x7b_tp4")


WORKLOADS = {
    "mlp_relu_tp2": mlp_relu_tp2,
    "mlp7b_tp4": mlp7b_tp4,
    "attn7b_tp4": attn7b_tp4,
    "layer70b_tp8": layer70b_tp8,
    "decode7b_tp2": decode7b_tp2,
    "mlp7b_tp4_fp8": mlp7b_tp4_fp8,
    "merge7b_tp4": merge7b_tp4,
    "backward7b_tp4": backward7b_tp4,
    "moe8x7b_tp4": moe8x7b_tp4,
}
