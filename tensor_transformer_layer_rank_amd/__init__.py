"""Python binding of libtpshard (one tensor-parallel rank's shard on an MI355X).

Argument marshalling only: every step runs in the HIP kernels of libtpshard.so,
reached through the C ABI declared in include/tpshard.h. Tensors are torch tensors on
the GPU (PyTorch provides device memory and the current stream). There is no CPU or
fallback path: if the library is missing, importing the entry points raises.

Names follow the C calls: column_linear, row_linear_partial, mlp_shard, attn_shard,
partial_sum (+ workspace-size queries and kernel timing).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "TpError", "lib", "load", "LIB_PATH", "column_linear", "row_linear_partial", "mlp_shard",
    "attn_shard", "partial_sum", "linear_workspace_size", "mlp_workspace_size",
    "attn_workspace_size", "mlp_shard_fp8", "mlp_fp8_workspace_size", "AttnDesc",
    "profile_enable", "profile_reset", "profile_read", "merge_rmsnorm", "linear_backward",
    "linear_backward_workspace_size", "moe_mlp_shard", "moe_workspace_size",
    "TP_F32", "TP_BF16", "TP_F16", "TP_FP8_E4M3", "TP_ACT_NONE", "TP_ACT_RELU",
    "TP_MLP_RELU", "TP_MLP_SWIGLU", "STATUS", "decode_step", "decode_step_workspace_size", "pack_strips",
    "column_linear_noalloc", "mfma_rate_probe", "hbm_read_probe",
]

# TPSHARD_LIB names another build of the same library (e.g. the host-checked one)
LIB_PATH = os.environ.get("TPSHARD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")

TP_F32, TP_BF16, TP_F16, TP_FP8_E4M3 = 0, 1, 2, 3
TP_ACT_NONE, TP_ACT_RELU = 0, 1
TP_MLP_RELU, TP_MLP_SWIGLU = 0, 1
STATUS = {0: "TP_OK", 1: "TP_ERR_NULL_POINTER", 2: "TP_ERR_BAD_SHAPE", 3: "TP_ERR_BAD_DTYPE",
          4: "TP_ERR_MISALIGNED", 5: "TP_ERR_WORKSPACE", 6: "TP_ERR_UNSUPPORTED", 7: "TP_ERR_HIP"}

EXPORTS = [
    "tp_column_linear", "tp_row_linear_partial", "tp_linear_workspace_size", "tp_mlp_shard",
    "tp_mlp_workspace_size", "tp_attn_shard", "tp_attn_workspace_size", "tp_partial_sum",
    "tp_status_string", "tp_last_error", "tp_abi_version", "tp_profile_enable",
    "tp_profile_read", "tp_profile_reset", "tp_mlp_shard_fp8", "tp_mlp_fp8_workspace_size",
    "tp_merge_rmsnorm", "tp_linear_backward", "tp_linear_backward_workspace_size", "tp_moe_mlp_shard",
    "tp_moe_workspace_size", "tp_column_linear_noalloc", "tp_mfma_rate_probe", "tp_decode_step",
    "tp_decode_step_workspace_size", "tp_decode_step_packed", "tp_pack_strips", "tp_packed_strips_bytes",
    "tp_hbm_read_probe",
]


class TpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("H", ctypes.c_int64),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_theta", ctypes.c_float), ("causal", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("cache_len", ctypes.c_int64), ("cache_capacity", ctypes.c_int64),
    ]


class Fp8Scales(ctypes.Structure):
    _fields_ = [("x_scale", ctypes.c_float), ("w_scale", ctypes.c_float)]


class Fp8MlpScales(ctypes.Structure):
    _fields_ = [("x_scale", ctypes.c_float), ("w_gate_scale", ctypes.c_float),
                ("w_up_scale", ctypes.c_float), ("w_down_scale", ctypes.c_float),
                ("h_scale", ctypes.c_float)]


_lib = None
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libtpshard.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"libtpshard.so not built at {path}; run "
                          "`python -m tensor_transformer_layer_rank_amd.build` first")
    L = ctypes.CDLL(path)
    sig = {
        "tp_column_linear": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _SZ, _P], _I32),
        "tp_row_linear_partial": ([_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P], _I32),
        "tp_linear_workspace_size": ([_I64, _I64, _I64, _I32], _SZ),
        "tp_mlp_shard": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _SZ, _P], _I32),
        "tp_mlp_workspace_size": ([_I64, _I64, _I64, _I32, _I32, _I32], _SZ),
        "tp_attn_shard": ([_P, _P, _P, _P, ctypes.POINTER(AttnDesc), _I32, _P, _SZ, _P], _I32),
        "tp_attn_workspace_size": ([ctypes.POINTER(AttnDesc), _I32], _SZ),
        "tp_partial_sum": ([ctypes.POINTER(_P), _I32, _P, _I64, _P], _I32),
        "tp_status_string": ([_I32], ctypes.c_char_p),
        "tp_last_error": ([], ctypes.c_char_p),
        "tp_abi_version": ([], ctypes.c_int),
        "tp_profile_enable": ([ctypes.c_int], _I32),
        "tp_profile_read": ([ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)], _I32),
        "tp_profile_reset": ([], _I32),
        "tp_mlp_shard_fp8": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, ctypes.POINTER(Fp8MlpScales),
                              _P, _SZ, _P], _I32),
        "tp_mlp_fp8_workspace_size": ([_I64, _I64, _I64, _I32], _SZ),
        "tp_merge_rmsnorm": ([ctypes.POINTER(_P), _I32, _P, _P, ctypes.c_float, _P, _P, _I64, _I64, _P], _I32),
        "tp_linear_backward": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P], _I32),
        "tp_linear_backward_workspace_size": ([_I64, _I64, _I64], _SZ),
        "tp_moe_mlp_shard": ([_P, _I64, _I64, _I64, _I32, _P, _P, _P, ctypes.POINTER(_I64), _P, _I32, _P, _P, _P,
                              _P, _SZ, _P], _I32),
        "tp_moe_workspace_size": ([_I64, _I64, _I64, _I32, ctypes.POINTER(_I64)], _SZ),
        "tp_column_linear_noalloc": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P], _I32),
        "tp_mfma_rate_probe": ([_P, _P, _I64, _I64, _P], _I32),
        "tp_decode_step": ([_P, _P, _P, ctypes.POINTER(AttnDesc), _P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, _SZ,
                            _P], _I32),
        "tp_decode_step_workspace_size": ([ctypes.POINTER(AttnDesc), _I64, _I64], _SZ),
        "tp_decode_step_packed": ([_P, _P, _P, ctypes.POINTER(AttnDesc), _P, _P, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                   _SZ, _P], _I32),
        "tp_pack_strips": ([_P, _I64, _I64, _P, _P], _I32),
        "tp_packed_strips_bytes": ([_I64, _I64], _SZ),
        "tp_hbm_read_probe": ([_P, _I64, _I64, _P, _P], _I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def lib() -> ctypes.CDLL:
    return load()


def _check(st: int):
    if st != 0:
        raise TpError(st, lib().tp_last_error().decode())


# --- tensor helpers -------------------------------------------------------------------------

def _dt(t) -> int:
    """tp_dtype of a tensor; uint8 and float8_e4m3fn tensors hold OCP E4M3 codes."""
    import torch
    m = {torch.float32: TP_F32, torch.bfloat16: TP_BF16, torch.float16: TP_F16,
         torch.uint8: TP_FP8_E4M3, torch.float8_e4m3fn: TP_FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libtpshard takes GPU tensors")
    if not t.is_contiguous():
        raise ValueError("libtpshard takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, ws=None):
    import torch
    if nbytes == 0:
        return None, 0
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: {ws.numel() * ws.element_size()} < {nbytes}")
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# --- entry points (same names as the C calls) --------------------------------------------------

def linear_workspace_size(T: int, K: int, N: int, in_dt: int) -> int:
    return int(lib().tp_linear_workspace_size(T, K, N, in_dt))


def _scales(X, scales):
    """Fp8Scales for E4M3 operands (scales = (x_scale, w_scale)), else None."""
    if _dt(X) != TP_FP8_E4M3:
        return None
    if scales is None:
        raise ValueError("fp8 operands need scales=(x_scale, w_scale)")
    return ctypes.byref(Fp8Scales(float(scales[0]), float(scales[1])))


def column_linear(X, W, Y=None, act: int = TP_ACT_NONE, out_dtype=None, ldy: int | None = None,
                  scales=None, workspace=None, stream=None):
    """Y = act(X @ W) for this rank's column shard W [K, N]; returns Y ([T, ldy] if given).
    E4M3 operands (uint8 codes) take scales=(x_scale, w_scale); their output defaults to bf16."""
    import torch
    T, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError(f"X is [*, {K}] but W is [{K2}, *]")
    if Y is None:
        default = torch.bfloat16 if _dt(X) == TP_FP8_E4M3 else X.dtype
        Y = torch.empty((T, N), dtype=out_dtype or default, device=X.device)
    ldy = ldy if ldy is not None else Y.shape[-1]
    q = _scales(X, scales)
    ws, wsb = _workspace(linear_workspace_size(T, K, N, _dt(X)), X.device, workspace)
    _check(lib().tp_column_linear(_ptr(X), _ptr(W), ctypes.c_void_p(Y.data_ptr()), T, K, N, ldy,
                                  _dt(X), _dt(Y), act, q, _ptr(ws), wsb, _stream(stream)))
    return Y


def column_linear_noalloc(X, W, Y=None, act: int = TP_ACT_NONE, out_dtype=None, ldy: int | None = None,
                          scales=None, stream=None):
    """column_linear through tp_column_linear_noalloc: no workspace, the library's static scratch."""
    import torch
    T, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError(f"X is [*, {K}] but W is [{K2}, *]")
    if Y is None:
        default = torch.bfloat16 if _dt(X) == TP_FP8_E4M3 else X.dtype
        Y = torch.empty((T, N), dtype=out_dtype or default, device=X.device)
    ldy = ldy if ldy is not None else Y.shape[-1]
    q = _scales(X, scales)
    _check(lib().tp_column_linear_noalloc(_ptr(X), _ptr(W), ctypes.c_void_p(Y.data_ptr()), T, K, N, ldy,
                                          _dt(X), _dt(Y), act, q, _stream(stream)))
    return Y


def row_linear_partial(X, W, Y=None, accumulate: bool = False, scales=None, workspace=None, stream=None):
    """fp32 partial X_shard @ W_shard [K_shard, N] of a row-parallel layer (E4M3 operands:
    scales=(x_scale, w_scale))."""
    import torch
    T, K = X.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError(f"X is [*, {K}] but W is [{K2}, *]")
    if Y is None:
        Y = torch.empty((T, N), dtype=torch.float32, device=X.device)
    q = _scales(X, scales)
    ws, wsb = _workspace(linear_workspace_size(T, K, N, _dt(X)), X.device, workspace)
    _check(lib().tp_row_linear_partial(_ptr(X), _ptr(W), _ptr(Y), T, K, N, _dt(X), int(accumulate),
                                       q, _ptr(ws), wsb, _stream(stream)))
    return Y


def mlp_workspace_size(T: int, H: int, I: int, kind: int, in_dt: int, h_dt: int | None = None) -> int:
    h_dt = in_dt if h_dt is None else h_dt
    return int(lib().tp_mlp_workspace_size(T, H, I, kind, in_dt, h_dt))


def mlp_shard(X, W_gate, W_up, W_down, Y=None, kind: int = TP_MLP_SWIGLU, workspace=None, stream=None,
              h_dtype: int | None = None):
    """fp32 partial of this rank's MLP block (ReLU form: W_up=None). h_dtype: storage of the
    intermediate h (TP_BF16 by default for bf16 inputs, or TP_F16)."""
    import torch
    T, H = X.shape
    I = W_gate.shape[1]
    if Y is None:
        Y = torch.empty((T, H), dtype=torch.float32, device=X.device)
    dt = _dt(X)
    hdt = dt if h_dtype is None else h_dtype
    ws, wsb = _workspace(mlp_workspace_size(T, H, I, kind, dt, hdt), X.device, workspace)
    _check(lib().tp_mlp_shard(_ptr(X), _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Y), T, H, I,
                              kind, dt, hdt, _ptr(ws), wsb, _stream(stream)))
    return Y


def mlp_fp8_workspace_size(T: int, H: int, I: int, kind: int) -> int:
    return int(lib().tp_mlp_fp8_workspace_size(T, H, I, kind))


def mlp_shard_fp8(X, W_gate, W_up, W_down, scales, Y=None, kind: int = TP_MLP_SWIGLU, workspace=None,
                  stream=None):
    """fp32 partial of this rank's MLP block on E4M3 codes (uint8 tensors).
    scales = (x_scale, w_gate_scale, w_up_scale, w_down_scale, h_scale)."""
    import torch
    T, H = X.shape
    I = W_gate.shape[1]
    if Y is None:
        Y = torch.empty((T, H), dtype=torch.float32, device=X.device)
    q = Fp8MlpScales(*[float(v) for v in scales])
    ws, wsb = _workspace(mlp_fp8_workspace_size(T, H, I, kind), X.device, workspace)
    _check(lib().tp_mlp_shard_fp8(_ptr(X), _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Y), T, H, I,
                                  kind, ctypes.byref(q), _ptr(ws), wsb, _stream(stream)))
    return Y


def _desc(B, S, H, hq, hkv, theta=10000.0, k_cache=None, v_cache=None, cache_len=0, head_dim=128):
    d = AttnDesc()
    d.B, d.S, d.H = B, S, H
    d.n_q_heads, d.n_kv_heads, d.head_dim = hq, hkv, head_dim
    d.rope_theta, d.causal = theta, 1
    d.k_cache = k_cache.data_ptr() if k_cache is not None else None
    d.v_cache = v_cache.data_ptr() if v_cache is not None else None
    d.cache_len = cache_len
    d.cache_capacity = k_cache.shape[2] if k_cache is not None else 0
    return d


def attn_workspace_size(B, S, H, hq, hkv, theta=10000.0, k_cache=None, v_cache=None, cache_len=0) -> int:
    d = _desc(B, S, H, hq, hkv, theta, k_cache, v_cache, cache_len)
    return int(lib().tp_attn_workspace_size(ctypes.byref(d), TP_BF16))


def attn_shard(X, W_qkv, W_o, B: int, S: int, hq: int, hkv: int, theta: float = 10000.0,
               k_cache=None, v_cache=None, cache_len: int = 0, Y=None, workspace=None, stream=None):
    """fp32 partial of this rank's attention block (prefill, or decode when a cache is given)."""
    import torch
    T, H = X.shape
    if Y is None:
        Y = torch.empty((T, H), dtype=torch.float32, device=X.device)
    for c in (k_cache, v_cache):
        if c is not None and not c.is_contiguous():
            raise ValueError("caches must be contiguous")
    d = _desc(B, S, H, hq, hkv, theta, k_cache, v_cache, cache_len)
    nb = int(lib().tp_attn_workspace_size(ctypes.byref(d), _dt(X)))
    ws, wsb = _workspace(max(nb, 1), X.device, workspace)
    _check(lib().tp_attn_shard(_ptr(X), _ptr(W_qkv), _ptr(W_o), _ptr(Y), ctypes.byref(d), _dt(X),
                               _ptr(ws), wsb, _stream(stream)))
    return Y


def decode_step_workspace_size(B, H, hq, hkv, theta, k_cache, v_cache, cache_len, I, V) -> int:
    d = _desc(B, 1, H, hq, hkv, theta, k_cache, v_cache, cache_len)
    return int(lib().tp_decode_step_workspace_size(ctypes.byref(d), I, V))


def pack_strips(W, out=None, stream=None):
    """W [K, N] (bf16/fp16) -> its 128-column strips [ceil(N/128), K, 128] through tp_pack_strips."""
    import torch
    K, N = W.shape
    if out is None:
        out = torch.empty(((N + 127) // 128, K, 128), dtype=W.dtype, device=W.device)
    _check(lib().tp_pack_strips(_ptr(W), K, N, _ptr(out), _stream(stream)))
    return out


def decode_step(X, W_qkv, W_o, hq: int, hkv: int, theta: float, k_cache, v_cache, cache_len: int,
                W_gate, W_up, W_down, W_lm=None, Y_attn=None, Y_mlp=None, logits=None, workspace=None,
                stream=None, packed: bool = False, I: int = None, V: int = None):
    """One rank's decode step (attention shard with KV-cache append, MLP shard and the vocabulary-
    split head on the same X) through tp_decode_step; returns (Y_attn, Y_mlp, logits or None).
    packed=True: tp_decode_step_packed, every weight from pack_strips ([strips, K, 128]), with
    I (= I_shard) and V (= V_shard, 0 without W_lm) given."""
    import torch
    B, H = X.shape
    if not packed:
        I = W_gate.shape[1]
        V = W_lm.shape[1] if W_lm is not None else 0
    elif I is None or V is None:
        raise ValueError("decode_step(packed=True) needs I and V")
    Y_attn = Y_attn if Y_attn is not None else torch.empty((B, H), dtype=torch.float32, device=X.device)
    Y_mlp = Y_mlp if Y_mlp is not None else torch.empty((B, H), dtype=torch.float32, device=X.device)
    if V and logits is None:
        logits = torch.empty((B, V), dtype=torch.float32, device=X.device)
    d = _desc(B, 1, H, hq, hkv, theta, k_cache, v_cache, cache_len)
    nb = int(lib().tp_decode_step_workspace_size(ctypes.byref(d), I, V))
    ws, wsb = _workspace(nb, X.device, workspace)
    fn = lib().tp_decode_step_packed if packed else lib().tp_decode_step
    _check(fn(_ptr(X), _ptr(W_qkv), _ptr(W_o), ctypes.byref(d), _ptr(W_gate), _ptr(W_up), _ptr(W_down), I,
              _ptr(W_lm), V, _ptr(Y_attn), _ptr(Y_mlp), _ptr(logits) if V else None, _ptr(ws), wsb,
              _stream(stream)))
    return Y_attn, Y_mlp, logits


def partial_sum(partials, out=None, stream=None):
    """((P0 + P1) + P2) + ... for fp32 GPU tensors of equal size."""
    import torch
    k = len(partials)
    n = partials[0].numel()
    if out is None:
        out = torch.empty_like(partials[0])
    arr = (ctypes.c_void_p * k)(*[p.data_ptr() for p in partials])
    for p in partials:
        _ptr(p)
    _check(lib().tp_partial_sum(arr, k, _ptr(out), n, _stream(stream)))
    return out


def merge_rmsnorm(partials, residual, gamma, eps: float = 1e-5, residual_out=None, normed=None, stream=None):
    """r = residual + ((P0 + P1) + ...), returns (bf16(r), bf16(rms_norm(r) * gamma)).
    partials: fp32 [T, H] GPU tensors; residual bf16 [T, H]; gamma bf16 [H].
    residual_out may be residual (in-place)."""
    import torch
    T, H = residual.shape
    k = len(partials)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if normed is None:
        normed = torch.empty_like(residual)
    for p in partials:
        _ptr(p)
    arr = (ctypes.c_void_p * k)(*[p.data_ptr() for p in partials])
    _check(lib().tp_merge_rmsnorm(arr, k, _ptr(residual), _ptr(gamma), float(eps), _ptr(residual_out),
                                  _ptr(normed), T, H, _stream(stream)))
    return residual_out, normed


def linear_backward_workspace_size(T: int, K: int, N: int) -> int:
    return int(lib().tp_linear_backward_workspace_size(T, K, N))


def linear_backward(X, W, dY, dX=None, dW=None, workspace=None, stream=None):
    """(dX, dW) = (dY . W^T, X^T . dY) in fp32 for bf16 X [T, K], W [K, N], dY [T, N]."""
    import torch
    T, K = X.shape
    N = W.shape[1]
    if dX is None:
        dX = torch.empty((T, K), dtype=torch.float32, device=X.device)
    if dW is None:
        dW = torch.empty((K, N), dtype=torch.float32, device=X.device)
    need = linear_backward_workspace_size(T, K, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _check(lib().tp_linear_backward(_ptr(X), _ptr(W), _ptr(dY), _ptr(dX), _ptr(dW), T, K, N, TP_BF16,
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return dX, dW


def _offsets(expert_offsets):
    offs = [int(v) for v in expert_offsets]
    return (ctypes.c_int64 * len(offs))(*offs), len(offs) - 1


def moe_workspace_size(T: int, H: int, I: int, expert_offsets) -> int:
    arr, E = _offsets(expert_offsets)
    return int(lib().tp_moe_workspace_size(T, H, I, E, arr))


def moe_mlp_shard(X, W_gate, W_up, W_down, expert_offsets, row_token, token_rows, gates, Y=None,
                  workspace=None, stream=None):
    """fp32 partial of a top-k MoE MLP over local experts (bf16 X [T, H], W_gate/W_up [E, H, I],
    W_down [E, I, H]; expert_offsets: host sequence [E+1]; row_token int32 [R], token_rows
    int32 [T, k], gates fp32 [T, k] on the GPU)."""
    import torch
    T, H = X.shape
    E, _, I = W_gate.shape
    arr, E2 = _offsets(expert_offsets)
    if E2 != E:
        raise ValueError(f"expert_offsets has {E2 + 1} entries for {E} experts")
    k = token_rows.shape[1]
    if Y is None:
        Y = torch.empty((T, H), dtype=torch.float32, device=X.device)
    need = moe_workspace_size(T, H, I, expert_offsets)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    rt = _ptr(row_token) if row_token is not None and row_token.numel() else None
    _check(lib().tp_moe_mlp_shard(_ptr(X), T, H, I, E, _ptr(W_gate), _ptr(W_up), _ptr(W_down), arr, rt, k,
                                  _ptr(token_rows), _ptr(gates), _ptr(Y), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))
    return Y


# --- kernel timing ------------------------------------------------------------------------------

def hbm_read_probe(buf, bytes_per_workgroup: int, n_workgroups: int, out, stream=None):
    """HBM read-rate microbenchmark (measurement aid): see tp_hbm_read_probe."""
    _check(lib().tp_hbm_read_probe(_ptr(buf), int(bytes_per_workgroup), int(n_workgroups), _ptr(out),
                                   _stream(stream)))


def mfma_rate_probe(operands, out, n_workgroups: int, iters: int, stream=None):
    """Matrix-pipe rate microbenchmark (measurement aid): see tp_mfma_rate_probe."""
    _check(lib().tp_mfma_rate_probe(_ptr(operands), _ptr(out), int(n_workgroups), int(iters), _stream(stream)))
    return out


def profile_enable(on: bool = True):
    _check(lib().tp_profile_enable(int(on)))


def profile_reset():
    _check(lib().tp_profile_reset())


def profile_read(prefix: str = ""):
    """(total milliseconds, launch count) of recorded kernels whose name starts with prefix."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().tp_profile_read(prefix.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
