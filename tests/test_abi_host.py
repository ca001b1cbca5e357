"""Host-only checks of the C ABI (no GPU needed; no call reaches a kernel).

* libtpshard.so loads and exports every function include/tpshard.h declares.
* Every validation error path returns its status before any HIP call: the pointers
  passed here are fake (never dereferenced) and no stream is touched.
"""
import ctypes
import os
import re

import pytest

import tensor_transformer_layer_rank_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return tp.load()


def test_header_declares_the_calls():
    names = _declared()
    for n in ("tp_column_linear", "tp_row_linear_partial", "tp_mlp_shard", "tp_attn_shard", "tp_partial_sum"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in _declared():
        assert hasattr(L, n), f"{n} declared in tpshard.h but not exported"
    assert set(_declared()) <= set(tp.EXPORTS)


def test_abi_version_and_status_strings(L):
    assert L.tp_abi_version() == 1
    for code, name in tp.STATUS.items():
        assert L.tp_status_string(code).decode() == name


FAKE = ctypes.c_void_p(0x1000)         # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x1002)     # misaligned


def _st(x):
    return tp.STATUS[x]


def test_column_linear_validation(L):
    f = L.tp_column_linear
    assert _st(f(None, FAKE, FAKE, 4, 8, 8, 8, tp.TP_BF16, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_NULL_POINTER"
    assert "non-NULL" in L.tp_last_error().decode()
    assert _st(f(FAKE, FAKE, FAKE, 0, 8, 8, 8, tp.TP_BF16, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 4, tp.TP_BF16, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 8, tp.TP_BF16, tp.TP_BF16, 7, None, None, 0, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, FAKE, FAKE, 4, 12, 8, 8, tp.TP_BF16, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_MISALIGNED"
    assert _st(f(FAKE_ODD, FAKE, FAKE, 100, 8, 8, 8, tp.TP_BF16, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_MISALIGNED"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 8, tp.TP_F32, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_BAD_DTYPE"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 8, tp.TP_FP8_E4M3, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 8, 9, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_BAD_DTYPE"
    # decode-size bf16 needs a workspace
    assert _st(f(FAKE, FAKE, FAKE, 4, 64, 64, 64, tp.TP_BF16, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_WORKSPACE"


def test_fp8_linear_validation(L):
    q = ctypes.byref(tp.Fp8Scales(0.5, 0.25))
    col, row = L.tp_column_linear, L.tp_row_linear_partial
    ok = [FAKE, FAKE, FAKE, 64, 32, 32, 32, tp.TP_FP8_E4M3, tp.TP_BF16, 0, q, None, 0, None]
    bad = list(ok); bad[10] = ctypes.byref(tp.Fp8Scales(0.0, 1.0))
    assert _st(col(*bad)) == "TP_ERR_BAD_SHAPE"                      # non-positive scale
    bad = list(ok); bad[4] = 24
    assert _st(col(*bad)) == "TP_ERR_MISALIGNED"                     # K not a multiple of 16
    bad = list(ok); bad[5] = 40; bad[6] = 40
    assert _st(col(*bad)) == "TP_ERR_MISALIGNED"                     # N not a multiple of 16
    bad = list(ok); bad[0] = FAKE_ODD
    assert _st(col(*bad)) == "TP_ERR_MISALIGNED"
    bad = list(ok); bad[8] = tp.TP_FP8_E4M3
    assert _st(col(*bad)) == "TP_ERR_BAD_DTYPE"                      # no fp8 output
    assert _st(row(FAKE, FAKE, FAKE, 64, 32, 32, tp.TP_FP8_E4M3, 0, None, None, 0, None)) == "TP_ERR_NULL_POINTER"
    assert _st(row(FAKE, FAKE, FAKE, 64, 40, 32, tp.TP_FP8_E4M3, 0, q, None, 0, None)) == "TP_ERR_MISALIGNED"
    # a grid past one round of the device with enough K steps needs the split workspace (256
    # compute units assumed when no device is visible); a short K leaves it whole
    need = L.tp_linear_workspace_size(4200, 2048, 4096, tp.TP_FP8_E4M3)
    assert need > 0
    assert L.tp_linear_workspace_size(4200, 512, 4096, tp.TP_FP8_E4M3) == 0
    assert _st(row(FAKE, FAKE, FAKE, 4200, 2048, 4096, tp.TP_FP8_E4M3, 0, q, None, 0, None)) == "TP_ERR_WORKSPACE"


def test_fp8_mlp_validation(L):
    f = L.tp_mlp_shard_fp8
    q = tp.Fp8MlpScales(0.01, 0.001, 0.001, 0.001, 0.125)
    ws = L.tp_mlp_fp8_workspace_size(512, 256, 128, tp.TP_MLP_SWIGLU)
    assert ws >= 512 * 128
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 512, 256, 128, tp.TP_MLP_SWIGLU, ctypes.byref(q), FAKE, ws, None]
    bad = list(args); bad[9] = None
    assert _st(f(*bad)) == "TP_ERR_NULL_POINTER"
    bad = list(args); bad[2] = None
    assert _st(f(*bad)) == "TP_ERR_NULL_POINTER"                     # SwiGLU without W_up
    bad = list(args); bad[8] = tp.TP_MLP_RELU
    assert _st(f(*bad)) == "TP_ERR_BAD_SHAPE"                        # ReLU form with a W_up
    bad = list(args); bad[9] = ctypes.byref(tp.Fp8MlpScales(0.01, 0.001, 0.001, 0.001, 0.0))
    assert _st(f(*bad)) == "TP_ERR_BAD_SHAPE"                        # h_scale must be positive
    bad = list(args); bad[7] = 136
    assert _st(f(*bad)) == "TP_ERR_MISALIGNED"                       # I_shard not a multiple of 16
    bad = list(args); bad[11] = ws - 1
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"
    bad = list(args); bad[10] = None
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"


def test_linear_workspace_sizes(L):
    assert L.tp_linear_workspace_size(4096, 4096, 4096, tp.TP_BF16) == 0
    assert L.tp_linear_workspace_size(32, 4096, 16000, tp.TP_BF16) > 32 * 16000 * 4
    assert L.tp_linear_workspace_size(32, 4096, 16000, tp.TP_F32) == 0


def test_row_linear_validation(L):
    f = L.tp_row_linear_partial
    assert _st(f(FAKE, None, FAKE, 4, 8, 8, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE, FAKE, FAKE, 4, -8, 8, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 10, tp.TP_BF16, 0, None, None, 0, None)) == "TP_ERR_MISALIGNED"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 9, 0, None, None, 0, None)) == "TP_ERR_BAD_DTYPE"
    # fp16 operands are offered; a decode-size call needs its split workspace
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, tp.TP_F16, 0, None, None, 0, None)) == "TP_ERR_WORKSPACE"


def test_mlp_validation(L):
    f = L.tp_mlp_shard
    ws = L.tp_mlp_workspace_size(512, 256, 128, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16)
    assert ws >= 512 * 128 * 2
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 512, 256, 128, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16, FAKE, ws, None]
    bad = list(args); bad[2] = None
    assert _st(f(*bad)) == "TP_ERR_NULL_POINTER"            # SwiGLU without W_up
    bad = list(args); bad[8] = tp.TP_MLP_RELU
    assert _st(f(*bad)) == "TP_ERR_BAD_SHAPE"               # ReLU form with a W_up
    bad = list(args); bad[12] = ws - 1
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"
    bad = list(args); bad[11] = None
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"
    bad = list(args); bad[10] = tp.TP_F16
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"                       # fp16 h also holds W_down in fp16
    ws16 = L.tp_mlp_workspace_size(512, 256, 128, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_F16)
    assert ws16 >= ws + 256 * 128 * 2
    bad = list(args); bad[10] = tp.TP_FP8_E4M3
    assert _st(f(*bad)) == "TP_ERR_BAD_DTYPE"
    bad = list(args); bad[10] = tp.TP_F16; bad[5] = 64; bad[12] = 1 << 30
    assert _st(f(*bad)) == "TP_ERR_UNSUPPORTED"                     # fp16 h is a prefill-size option
    bad = list(args); bad[7] = 100
    bws = L.tp_mlp_workspace_size(512, 256, 100, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16)
    bad[12] = bws
    assert _st(f(*bad)) == "TP_ERR_MISALIGNED"              # I_shard not a multiple of 8
    bad = list(args); bad[5] = 0
    assert _st(f(*bad)) == "TP_ERR_BAD_SHAPE"
    # fp16 operands keep h in fp16 (any T); their workspace holds no converted W_down
    bad = list(args); bad[9] = tp.TP_F16
    assert _st(f(*bad)) == "TP_ERR_BAD_DTYPE"                       # fp16 input with a bf16 h
    assert L.tp_mlp_workspace_size(512, 256, 128, tp.TP_MLP_SWIGLU, tp.TP_F16, tp.TP_BF16) == 0
    w16 = L.tp_mlp_workspace_size(512, 256, 128, tp.TP_MLP_SWIGLU, tp.TP_F16, tp.TP_F16)
    assert w16 == ws
    assert L.tp_mlp_workspace_size(32, 256, 128, tp.TP_MLP_SWIGLU, tp.TP_F16, tp.TP_F16) > 0
    bad = list(args); bad[9] = tp.TP_F16; bad[10] = tp.TP_F16; bad[12] = w16 - 1
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"


def _desc(**kw):
    d = tp.AttnDesc()
    d.B, d.S, d.H, d.n_q_heads, d.n_kv_heads, d.head_dim = 2, 64, 256, 4, 2, 128
    d.rope_theta, d.causal = 10000.0, 1
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_attn_validation(L):
    f = L.tp_attn_shard
    def st(d, ws=1 << 30):
        return _st(f(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), tp.TP_BF16, FAKE, ws, None))
    assert st(_desc(head_dim=64)) == "TP_ERR_UNSUPPORTED"
    assert st(_desc(n_q_heads=3)) == "TP_ERR_BAD_SHAPE"
    assert st(_desc(causal=0)) == "TP_ERR_UNSUPPORTED"
    assert st(_desc(S=60)) == "TP_ERR_MISALIGNED"
    assert st(_desc(B=1 << 20, S=1 << 11)) == "TP_ERR_UNSUPPORTED"   # B*S = 2^31 tokens
    assert st(_desc(B=1, S=(1 << 24) + 8)) == "TP_ERR_UNSUPPORTED"   # S past 2^24
    assert st(_desc(k_cache=0x1000)) == "TP_ERR_NULL_POINTER"
    assert st(_desc(S=1, k_cache=0x1000, v_cache=0x2000, cache_len=8, cache_capacity=8)) == "TP_ERR_BAD_SHAPE"
    assert st(_desc(S=4, k_cache=0x1000, v_cache=0x2000, cache_len=2, cache_capacity=8)) == "TP_ERR_UNSUPPORTED"
    assert st(_desc(), ws=16) == "TP_ERR_WORKSPACE"
    assert _st(f(FAKE, FAKE, FAKE, FAKE, None, tp.TP_BF16, FAKE, 16, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE, FAKE, FAKE, FAKE, ctypes.byref(_desc()), tp.TP_F32, FAKE, 1 << 30, None)) == "TP_ERR_BAD_DTYPE"
    d = _desc()
    need = L.tp_attn_workspace_size(ctypes.byref(d), tp.TP_BF16)
    T = 2 * 64
    assert need >= T * (4 + 2 + 2 + 4) * 128 * 2          # q, k, vt, attention output
    dd = _desc(S=1, k_cache=0x1000, v_cache=0x2000, cache_len=100, cache_capacity=128)
    assert L.tp_attn_workspace_size(ctypes.byref(dd), tp.TP_BF16) > 0


def test_partial_sum_validation(L):
    f = L.tp_partial_sum
    arr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert _st(f(arr, 0, FAKE, 8, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(arr, 17, FAKE, 8, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(arr, 2, FAKE, 0, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(None, 2, FAKE, 8, None)) == "TP_ERR_NULL_POINTER"
    arr2 = (ctypes.c_void_p * 2)(0x1000, None)
    assert _st(f(arr2, 2, FAKE, 8, None)) == "TP_ERR_NULL_POINTER"
    arr3 = (ctypes.c_void_p * 2)(0x1000, 0x2004)
    assert _st(f(arr3, 2, FAKE, 8, None)) == "TP_ERR_MISALIGNED"


def test_merge_rmsnorm_validation(L):
    f = L.tp_merge_rmsnorm
    arr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    ok = (arr, 2, FAKE, FAKE, 1e-5, FAKE, FAKE, 4, 64, None)

    def st(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _st(f(*a))
    assert st(a1=0) == "TP_ERR_BAD_SHAPE" and st(a1=17) == "TP_ERR_BAD_SHAPE"
    assert st(a0=None) == "TP_ERR_NULL_POINTER"
    assert st(a0=(ctypes.c_void_p * 2)(0x1000, None)) == "TP_ERR_NULL_POINTER"
    for i in (2, 3, 5, 6):
        assert st(**{f"a{i}": None}) == "TP_ERR_NULL_POINTER"
        assert st(**{f"a{i}": FAKE_ODD}) == "TP_ERR_MISALIGNED"
    assert st(a0=(ctypes.c_void_p * 2)(0x1000, 0x2004)) == "TP_ERR_MISALIGNED"
    assert st(a7=0) == "TP_ERR_BAD_SHAPE" and st(a8=0) == "TP_ERR_BAD_SHAPE"
    assert st(a8=60) == "TP_ERR_UNSUPPORTED"                      # H % 8
    assert st(a8=16384 + 8) == "TP_ERR_UNSUPPORTED"               # H past 16384
    assert st(a7=1 << 31) == "TP_ERR_UNSUPPORTED"                 # T rows
    assert st(a4=-1.0) == "TP_ERR_BAD_SHAPE" and st(a4=float("nan")) == "TP_ERR_BAD_SHAPE"
    assert st(a4=float("inf")) == "TP_ERR_BAD_SHAPE"


def test_linear_backward_validation(L):
    f = L.tp_linear_backward
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 128, 256, tp.TP_BF16, FAKE, 1 << 30, None]

    def st(i, v):
        a = list(ok)
        a[i] = v
        return _st(f(*a))
    for i in range(5):
        assert st(i, None) == "TP_ERR_NULL_POINTER"
        assert st(i, FAKE_ODD) == "TP_ERR_MISALIGNED"
    assert st(8, tp.TP_F32) == "TP_ERR_BAD_DTYPE"
    for i in (5, 6, 7):
        assert st(i, 0) == "TP_ERR_BAD_SHAPE"
        assert st(i, 60) == "TP_ERR_MISALIGNED"
        assert st(i, 1 << 23) == "TP_ERR_UNSUPPORTED"
    assert st(10, 16) == "TP_ERR_WORKSPACE"
    assert st(9, None) == "TP_ERR_WORKSPACE"
    need = L.tp_linear_backward_workspace_size(64, 128, 256)
    assert need > 0 and need % 256 == 0                              # split-K partials of the small grids
    # W and X are read in place: grids of whole rounds need no workspace at all
    assert L.tp_linear_backward_workspace_size(4096, 4096, 4096) == 0


def test_moe_validation(L):
    f = L.tp_moe_mlp_shard
    offs = (ctypes.c_int64 * 3)(0, 4, 8)
    ok = [FAKE, 4, 64, 32, 2, FAKE, FAKE, FAKE, offs, FAKE, 2, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]

    def st(i, v):
        a = list(ok)
        a[i] = v
        return _st(f(*a))
    for i in (0, 5, 6, 7, 8, 11, 12, 13):
        assert st(i, None) == "TP_ERR_NULL_POINTER", i
    assert st(9, None) == "TP_ERR_NULL_POINTER"                       # rows exist
    for i in (1, 2, 3):
        assert st(i, 0) == "TP_ERR_BAD_SHAPE"
    assert st(4, 0) == "TP_ERR_BAD_SHAPE" and st(4, 1025) == "TP_ERR_BAD_SHAPE"
    assert st(10, 0) == "TP_ERR_BAD_SHAPE" and st(10, 17) == "TP_ERR_BAD_SHAPE"
    assert st(8, (ctypes.c_int64 * 3)(1, 4, 8)) == "TP_ERR_BAD_SHAPE"  # offsets must start at 0
    assert st(8, (ctypes.c_int64 * 3)(0, 4, 2)) == "TP_ERR_BAD_SHAPE"  # and not decrease
    assert st(2, 60) == "TP_ERR_MISALIGNED" and st(3, 36) == "TP_ERR_MISALIGNED"
    for i in (0, 5, 6, 7, 13):
        assert st(i, FAKE_ODD) == "TP_ERR_MISALIGNED", i
    assert st(12, ctypes.c_void_p(0x1002)) == "TP_ERR_MISALIGNED"
    assert st(15, 16) == "TP_ERR_WORKSPACE" and st(14, None) == "TP_ERR_WORKSPACE"
    need = L.tp_moe_workspace_size(4, 64, 32, 2, offs)
    assert need >= 8 * 64 * (2 + 4)
    assert L.tp_moe_workspace_size(4, 64, 32, 2, (ctypes.c_int64 * 3)(0, 5, 2)) == 0
    # experts of more than 64 rows take the grouped GEMMs: h for every row joins the workspace
    big = (ctypes.c_int64 * 3)(0, 100, 300)
    assert L.tp_moe_workspace_size(200, 64, 32, 2, big) >= 300 * 64 * (2 + 4) + 300 * 32 * 2
    # a grouped launch past 2^28 tiles is refused before anything runs
    a = list(ok)
    a[1], a[2], a[4], a[8] = 1 << 30, 8192, 1, (ctypes.c_int64 * 2)(0, 1 << 30)
    assert _st(f(*a)) == "TP_ERR_UNSUPPORTED"


def test_profile_api_without_launches(L):
    assert L.tp_profile_reset() == 0
    ms, n = tp.profile_read("")
    assert ms == 0.0 and n == 0


def test_fp16_operands_follow_the_bf16_rules(L):
    col, row = L.tp_column_linear, L.tp_row_linear_partial
    assert L.tp_linear_workspace_size(32, 4096, 16000, tp.TP_F16) == L.tp_linear_workspace_size(32, 4096, 16000, tp.TP_BF16)
    assert _st(col(FAKE, FAKE, FAKE, 100, 12, 8, 8, tp.TP_F16, tp.TP_F32, 0, None, None, 0, None)) == "TP_ERR_MISALIGNED"
    assert _st(col(FAKE_ODD, FAKE, FAKE, 100, 8, 8, 8, tp.TP_F16, tp.TP_F16, 0, None, None, 0, None)) == "TP_ERR_MISALIGNED"
    # the few-row regime offers every output type too: an fp16-output call passes the dtype checks
    # and stops at the workspace size (no launch with these fake pointers)
    assert _st(col(FAKE, FAKE, FAKE, 4, 64, 64, 64, tp.TP_F16, tp.TP_F16, 0, None, FAKE, 16, None)) == "TP_ERR_WORKSPACE"
    assert _st(col(FAKE, FAKE, FAKE, 4, 64, 64, 64, tp.TP_BF16, tp.TP_F32, 1, None, FAKE, 16, None)) == "TP_ERR_WORKSPACE"
    assert _st(row(FAKE, FAKE, FAKE, 100, 12, 8, tp.TP_F16, 0, None, None, 0, None)) == "TP_ERR_MISALIGNED"


def test_contraction_lengths_past_2_pow_23_are_refused(L):
    """The MFMA tiles address a 256-row activation block with 32-bit offsets (row * lda), so every
    16-bit / fp8 GEMM entry point refuses an activation row length of 2^23 elements or more before
    any launch (the pointers here are fake and never touched)."""
    big = 1 << 23
    q = ctypes.byref(tp.Fp8Scales(0.5, 0.25))
    col, row = L.tp_column_linear, L.tp_row_linear_partial
    for dt, qq in ((tp.TP_BF16, None), (tp.TP_F16, None), (tp.TP_FP8_E4M3, q)):
        assert _st(col(FAKE, FAKE, FAKE, 512, big, 64, 64, dt, tp.TP_F32, 0, qq, FAKE, 1 << 40, None)) == "TP_ERR_UNSUPPORTED"
        assert _st(row(FAKE, FAKE, FAKE, 512, big, 64, dt, 0, qq, FAKE, 1 << 40, None)) == "TP_ERR_UNSUPPORTED"
        assert "2^23" in L.tp_last_error().decode()
    mlp = L.tp_mlp_shard
    assert _st(mlp(FAKE, FAKE, FAKE, FAKE, FAKE, 512, big, 64, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16, FAKE,
                   1 << 40, None)) == "TP_ERR_UNSUPPORTED"
    assert _st(mlp(FAKE, FAKE, FAKE, FAKE, FAKE, 512, 64, big, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16, FAKE,
                   1 << 40, None)) == "TP_ERR_UNSUPPORTED"
    fq = ctypes.byref(tp.Fp8MlpScales(0.01, 0.001, 0.001, 0.001, 0.125))
    assert _st(L.tp_mlp_shard_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 512, big, 64, tp.TP_MLP_SWIGLU, fq, FAKE, 1 << 40,
                                  None)) == "TP_ERR_UNSUPPORTED"
    d = tp._desc(1, 256, big, 8, 8)
    assert _st(L.tp_attn_shard(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), tp.TP_BF16, FAKE, 1 << 40, None)) == \
        "TP_ERR_UNSUPPORTED"
    offs = (ctypes.c_int64 * 2)(0, 300)
    assert _st(L.tp_moe_mlp_shard(FAKE, 300, big, 64, 1, FAKE, FAKE, FAKE, offs, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None)) == "TP_ERR_UNSUPPORTED"


def test_backward_grid_limit(L):
    """2^23 - 8 in two dimensions would need about 2^30 GEMM tiles: refused before launch."""
    n = (1 << 23) - 8
    assert _st(L.tp_linear_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 64, n, n, tp.TP_BF16, FAKE, 1 << 40, None)) == \
        "TP_ERR_UNSUPPORTED"
    assert "2^22 tiles" in L.tp_last_error().decode()


def test_noalloc_column_linear_validation(L):
    """The allocation-free variant checks like tp_column_linear and refuses a few-row call whose
    partial sums exceed its static scratch, before any HIP call."""
    f = L.tp_column_linear_noalloc
    assert _st(f(None, FAKE, FAKE, 4, 8, 8, 8, tp.TP_BF16, tp.TP_BF16, 0, None, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE, FAKE, FAKE, 4, 12, 8, 8, tp.TP_BF16, tp.TP_BF16, 0, None, None)) == "TP_ERR_MISALIGNED"
    assert _st(f(FAKE, FAKE, FAKE, 4, 8, 8, 8, 9, tp.TP_BF16, 0, None, None)) == "TP_ERR_BAD_DTYPE"
    assert L.tp_linear_workspace_size(64, 512, 131072, tp.TP_BF16) > 16 << 20
    assert _st(f(FAKE, FAKE, FAKE, 64, 512, 131072, 131072, tp.TP_BF16, tp.TP_F32, 0, None, None)) == "TP_ERR_UNSUPPORTED"
    assert "scratch" in L.tp_last_error().decode()


def test_mfma_rate_probe_validation(L):
    f = L.tp_mfma_rate_probe
    assert _st(f(None, FAKE, 256, 100, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE_ODD, FAKE, 256, 100, None)) == "TP_ERR_MISALIGNED"
    assert _st(f(FAKE, FAKE, 0, 100, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, FAKE, 256, 0, None)) == "TP_ERR_BAD_SHAPE"


def test_hbm_read_probe_validation(L):
    f = L.tp_hbm_read_probe
    assert _st(f(None, 8192, 4, FAKE, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE, 8192, 4, None, None)) == "TP_ERR_NULL_POINTER"
    assert _st(f(FAKE_ODD, 8192, 4, FAKE, None)) == "TP_ERR_MISALIGNED"
    assert _st(f(FAKE, 8192 + 16, 4, FAKE, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, 4096, 4, FAKE, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, 8192, 0, FAKE, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(f(FAKE, 8192, (1 << 20) + 1, FAKE, None)) == "TP_ERR_BAD_SHAPE"


def test_decode_step_validation(L):
    f = L.tp_decode_step
    d = tp._desc(4, 8, 256, 2, 2)          # no cache: a prefill, not a decode step
    args = [FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, 136, FAKE, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    assert _st(f(*args)) == "TP_ERR_BAD_SHAPE"
    d = tp.AttnDesc()
    d.B, d.S, d.H, d.n_q_heads, d.n_kv_heads, d.head_dim, d.rope_theta, d.causal = 4, 1, 256, 2, 2, 128, 1e4, 1
    d.k_cache, d.v_cache, d.cache_len, d.cache_capacity = 0x1000, 0x2000, 37, 40
    args[3] = ctypes.byref(d)
    assert L.tp_decode_step_workspace_size(ctypes.byref(d), 136, 1000) > 0
    assert L.tp_decode_step_workspace_size(ctypes.byref(d), 136, 0) > 0
    bad = list(args); bad[0] = None
    assert _st(f(*bad)) == "TP_ERR_NULL_POINTER"
    bad = list(args); bad[12] = None
    assert _st(f(*bad)) == "TP_ERR_NULL_POINTER"                      # logits needed for V_shard > 0
    bad = list(args); bad[8] = None
    assert _st(f(*bad)) == "TP_ERR_BAD_SHAPE"                         # V_shard > 0 without W_lm
    bad = list(args); bad[7] = 132
    assert _st(f(*bad)) == "TP_ERR_MISALIGNED"                        # I_shard not a multiple of 8
    bad = list(args); bad[14] = 16
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"
    bad = list(args); bad[6] = FAKE_ODD
    assert _st(f(*bad)) == "TP_ERR_MISALIGNED"
    d.B = 65
    assert _st(f(*args)) == "TP_ERR_UNSUPPORTED"                      # at most 64 sequences


def test_packed_decode_validation(L):
    """tp_decode_step_packed validates like tp_decode_step; tp_pack_strips and its size query
    reject NULL, misaligned and unpackable arguments before any HIP call."""
    f = L.tp_decode_step_packed
    d = tp.AttnDesc()
    d.B, d.S, d.H, d.n_q_heads, d.n_kv_heads, d.head_dim, d.rope_theta, d.causal = 4, 1, 256, 2, 2, 128, 1e4, 1
    d.k_cache, d.v_cache, d.cache_len, d.cache_capacity = 0x1000, 0x2000, 37, 40
    args = [FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, FAKE, FAKE, 136, FAKE, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    bad = list(args); bad[1] = None
    assert _st(f(*bad)) == "TP_ERR_NULL_POINTER"
    assert "tp_decode_step_packed" in L.tp_last_error().decode()
    bad = list(args); bad[14] = 16
    assert _st(f(*bad)) == "TP_ERR_WORKSPACE"
    bad = list(args); bad[7] = 132
    assert _st(f(*bad)) == "TP_ERR_MISALIGNED"
    g = L.tp_pack_strips
    assert _st(g(None, 64, 256, FAKE, None)) == "TP_ERR_NULL_POINTER"
    assert _st(g(FAKE, 64, 256, None, None)) == "TP_ERR_NULL_POINTER"
    assert _st(g(FAKE, 0, 256, FAKE, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(g(FAKE, 64, 0, FAKE, None)) == "TP_ERR_BAD_SHAPE"
    assert _st(g(FAKE, 64, 252, FAKE, None)) == "TP_ERR_MISALIGNED"
    assert _st(g(FAKE_ODD, 64, 256, FAKE, None)) == "TP_ERR_MISALIGNED"
    assert _st(g(FAKE, 1 << 40, 256, FAKE, None)) == "TP_ERR_UNSUPPORTED"
    assert _st(g(FAKE, 1 << 20, 1 << 20, FAKE, None)) == "TP_ERR_UNSUPPORTED"   # 2^40 elements
    assert L.tp_packed_strips_bytes(1 << 20, 1 << 20) == 0
    assert L.tp_packed_strips_bytes(1 << 20, 1 << 16) == (1 << 36) * 2       # exactly 2^36 elements
    assert L.tp_packed_strips_bytes(4096, 16000) == 125 * 4096 * 128 * 2
    assert L.tp_packed_strips_bytes(40, 136) == 2 * 40 * 128 * 2
    assert L.tp_packed_strips_bytes(40, 132) == 0
    assert L.tp_packed_strips_bytes(0, 128) == 0


def test_workspace_size_arithmetic_at_large_shapes(L):
    """Every size query at large valid shapes: positive, in range, and growing with the token
    count (run under the host-sanitizer build, this also checks the size arithmetic for
    signed overflow and out-of-bounds host accesses)."""
    big = 1 << 62
    for T in (64, 1 << 16, 1 << 22):
        assert 0 < L.tp_linear_workspace_size(32, (1 << 23) - 8, 1 << 16, tp.TP_BF16) < big
        assert L.tp_linear_workspace_size(T, 16384, 53248, tp.TP_BF16) < big
        m1 = L.tp_mlp_workspace_size(T, 16384, 53248, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16)
        m2 = L.tp_mlp_workspace_size(2 * T, 16384, 53248, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_BF16)
        assert 0 < m1 < m2 < big
        if T > 64:
            assert m1 < L.tp_mlp_workspace_size(T, 16384, 53248, tp.TP_MLP_SWIGLU, tp.TP_BF16, tp.TP_F16) < big
        assert 0 < L.tp_mlp_fp8_workspace_size(T, 16384, 53248, tp.TP_MLP_SWIGLU) < big
        assert L.tp_linear_backward_workspace_size(T, 8192, 8192) < big
    for B, S in ((1, 1 << 20), (64, 1 << 14), (1 << 12, 1 << 8)):
        d = _desc(B=B, S=S, H=16384, n_q_heads=64, n_kv_heads=8)
        assert 0 < L.tp_attn_workspace_size(ctypes.byref(d), tp.TP_BF16) < big
    d = _desc(B=64, S=1, H=16384, n_q_heads=128, n_kv_heads=16, k_cache=0x1000, v_cache=0x2000,
              cache_len=(1 << 20) - 1, cache_capacity=1 << 20)
    assert 0 < L.tp_decode_step_workspace_size(ctypes.byref(d), 53248, 128000) < big
    E = 64
    offs = (ctypes.c_int64 * (E + 1))(*[i * (1 << 14) for i in range(E + 1)])
    assert 0 < L.tp_moe_workspace_size(1 << 19, 8192, 16384, E, offs) < big
