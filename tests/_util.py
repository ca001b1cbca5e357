"""Helpers shared by the test modules (no arithmetic of the method lives here)."""
import numpy as np

from workloads.device import codes_to_device as dev_codes, to_device as dev, to_host as host  # noqa: F401

# (what, relF, max-abs) of every comparison made through assert_close_bf16 in this session;
# conftest.py prints them at the end of the run
PARITY_LOG = []

REL_F_TOL = 5e-3     # relative Frobenius error bound for bf16 inputs with fp32 accumulation
MAX_ABS_TOL = 3e-2   # max-abs error bound for the same


def rel_fro(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


OUT_ROUNDING = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def assert_close_bf16(got, ref, what="", out="f32"):
    """relF <= 5e-3 and max-abs <= 3e-2 (fp32 outputs).

    For outputs stored in bf16/fp16 the rounding of the stored value itself (half an
    ulp: 2^-8 resp. 2^-11 of |ref|) is added to the max-abs bound: the storage format
    cannot hold the exact value, and the tolerance applies to the arithmetic before it.
    Returns (relF, max-abs beyond that allowance); the raw max-abs is logged too.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rf = rel_fro(got, ref)
    diff = np.abs(got - ref)
    err = diff - OUT_ROUNDING[out] * np.abs(ref)
    ma = float(np.max(err))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    PARITY_LOG.append((what, rf, float(np.max(diff)), ma, got.size))
    assert rf <= REL_F_TOL and ma <= MAX_ABS_TOL, f"{what}: relF={rf:.3e} max-abs={ma:.3e}"
    return rf, ma


def sample_rows(T: int, n: int, seed: int = 0):
    """First, last and random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = set([0, T - 1]) | set(rng.integers(0, T, size=n).tolist())
    return np.array(sorted(rows), dtype=np.int64)


