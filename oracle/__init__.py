"""Python access to the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the GPU library never does.  Every function
takes and returns numpy arrays in the storage formats of the synth package
(int8 codes, uint16 fp16/bf16 bit patterns, int64 targets).

The oracle is pinned by the `-m "not gpu"` tests in tests/test_oracle_*.py
(closed forms, exact rational sums, brute force, algebraic invariants and
high-precision decimal references), never by the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of the oracle (the mutation test does).
_LIB_OVERRIDE = os.environ.get("W8INV_ORACLE_LIB")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        P, I64, U32, F32, F64, I32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32,
                                      ctypes.c_float, ctypes.c_double, ctypes.c_int)
        L.oracle_w8_linear.argtypes = [P, P, P, I64, I64, I64, I64, P, I64, P, P]
        L.oracle_block_logprob.argtypes = [P, P, I64, I64, I64, I64, P, P, I32]
        L.oracle_argmax.argtypes = [P, I64, I64, I64, P]
        L.oracle_logprob_ref.argtypes = [P, P, I64, I64, I64, P]
        L.oracle_exp32.argtypes, L.oracle_exp32.restype = [F32], F32
        L.oracle_log32.argtypes, L.oracle_log32.restype = [F32], F32
        L.oracle_exp32_array.argtypes = [P, I64, P]
        L.oracle_log32_array.argtypes = [P, I64, P]
        L.oracle_exp32_bits.argtypes = [U32, I64, P]
        L.oracle_log32_bits.argtypes = [U32, I64, P]
        L.oracle_bf16_round.argtypes, L.oracle_bf16_round.restype = [F64], ctypes.c_uint16
        L.oracle_bf16_value.argtypes, L.oracle_bf16_value.restype = [ctypes.c_uint16], F64
        L.oracle_f16_value.argtypes, L.oracle_f16_value.restype = [ctypes.c_uint16], F64
        L.oracle_max_threads.restype = I32
        L.oracle_rmsnorm.argtypes = [P, P, F64, I64, I64, I64, P]
        L.oracle_swiglu.argtypes = [P, I64, I64, I64, P]
        L.oracle_add.argtypes = [P, P, I64, I64, I64, I64, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def w8_linear(q, s, x, rows=None, mass: bool = False):
    """fp64 y[t, len(rows)] = dequant(W)[rows] . x^T  (x is [t, K] bf16 bits).

    mass=True returns (y, m) with m the absolute sums sum_k |q s x| of the same terms."""
    q = _c(q, np.int8)
    s = _c(s, np.uint16)
    x = _c(x, np.uint16)
    N, K = q.shape
    t = x.shape[0]
    assert x.shape[1] == K and s.shape == (N, K // 32)
    if rows is None:
        nrows, rp = N, None
    else:
        rows = _c(rows, np.int64)
        assert rows.min(initial=0) >= 0 and rows.max(initial=0) < N
        nrows, rp = rows.size, _ptr(rows)
    y = np.empty((t, nrows), dtype=np.float64)
    m = np.empty((t, nrows), dtype=np.float64) if mass else None
    if t and nrows:
        lib().oracle_w8_linear(_ptr(q), _ptr(s), _ptr(x), N, K, t, K, rp, nrows, _ptr(y),
                               _ptr(m) if mass else None)
    return (y, m) if mass else y


def block_logprob(logits, targets, block: int, return_partials: bool = False, direct: bool = False):
    """Fixed-order fp32 target logprob over `block`-wide vocabulary blocks; fp32 [t].

    direct=False: the blockwise form -(log(sum_exp) - target); True: blockwise-direct,
    target - log(sum_exp) (tokenspeed numerics, "Logprobs")."""
    logits = _c(logits, np.uint16)
    targets = _c(targets, np.int64)
    t, V = logits.shape
    nb = (V + block - 1) // block
    out = np.empty(t, dtype=np.float32)
    part = np.empty((t, nb), dtype=np.float32) if return_partials else None
    if t:
        lib().oracle_block_logprob(_ptr(logits), _ptr(targets), block, t, V, V, _ptr(out),
                                   _ptr(part) if part is not None else None, 1 if direct else 0)
    return (out, part) if return_partials else out


def argmax(logits) -> np.ndarray:
    """Canonical greedy argmax per column: the maximum, lowest index on ties, +-0 equal, the first
    NaN when there is one (tokenspeed numerics, "Logprobs"); int64 [t]."""
    logits = _c(logits, np.uint16)
    t, V = logits.shape
    out = np.empty(t, dtype=np.int64)
    if t:
        lib().oracle_argmax(_ptr(logits), t, V, V, _ptr(out))
    return out


def logprob_ref(logits, targets) -> np.ndarray:
    """Extended-precision (long double) target logprob, as float64 [t]."""
    logits = _c(logits, np.uint16)
    targets = _c(targets, np.int64)
    t, V = logits.shape
    out = np.empty(t, dtype=np.float64)
    if t:
        lib().oracle_logprob_ref(_ptr(logits), _ptr(targets), t, V, V, _ptr(out))
    return out


def exp32(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    lib().oracle_exp32_array(_ptr(x), x.size, _ptr(out))
    return out


def log32(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    lib().oracle_log32_array(_ptr(x), x.size, _ptr(out))
    return out


def exp32_bits(start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    lib().oracle_exp32_bits(start, count, _ptr(out))
    return out


def log32_bits(start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    lib().oracle_log32_bits(start, count, _ptr(out))
    return out


def bf16_round(v: float) -> int:
    return int(lib().oracle_bf16_round(float(v)))


def bf16_round_array(a) -> np.ndarray:
    f = lib().oracle_bf16_round
    a = np.asarray(a, dtype=np.float64)
    return np.fromiter((f(float(v)) for v in a.ravel()), dtype=np.uint16, count=a.size).reshape(a.shape)


def bf16_value(b: int) -> float:
    return float(lib().oracle_bf16_value(int(b)))


def f16_value(h: int) -> float:
    return float(lib().oracle_f16_value(int(h)))


def rmsnorm(x, eps: float, weight=None) -> np.ndarray:
    x = _c(x, np.uint16)
    t, H = x.shape
    y = np.empty((t, H), dtype=np.float64)
    w = _c(weight, np.uint16) if weight is not None else None
    lib().oracle_rmsnorm(_ptr(x), _ptr(w) if w is not None else None, eps, t, H, H, _ptr(y))
    return y


def swiglu(gu) -> np.ndarray:
    gu = _c(gu, np.uint16)
    t, F2 = gu.shape
    F = F2 // 2
    y = np.empty((t, F), dtype=np.float64)
    lib().oracle_swiglu(_ptr(gu), t, F, F2, _ptr(y))
    return y


def add(a, b) -> np.ndarray:
    a = _c(a, np.uint16)
    b = _c(b, np.uint16)
    t, H = a.shape
    y = np.empty((t, H), dtype=np.float64)
    lib().oracle_add(_ptr(a), _ptr(b), t, H, H, H, _ptr(y))
    return y
