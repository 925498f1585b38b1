"""CPU oracle for the skinny W4A8/W6A8 linear (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library.

The arithmetic lives in ``oracle.c`` (plain loops, OpenMP over output rows);
this module builds it with gcc when the shared object is missing or stale and
wraps it with ctypes.  ``layer_sequence`` composes those calls into the
decode-step walk of the "Doubling LLM token rates in ComfyUI" page (section
"What is the bottleneck?": every step reads every weight matrix once; section
"Optimizing the Linear Kernel": the quantisation absorbs the RMSNorm that
precedes it).  Function-level readings are stated in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
GROUP = 128

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_decode.argtypes = [ctypes.c_int, I64, I64, P, P]
        lib.oracle_quantize_act.argtypes = [I64, I64, P, P, P]
        lib.oracle_rmsnorm_bf16.argtypes = [I64, I64, P, P]
        lib.oracle_wrmsnorm_bf16.argtypes = [I64, I64, P, P, P]
        lib.oracle_swiglu_bf16.argtypes = [I64, P, P, P]
        lib.oracle_decode_attention.argtypes = [I64, I64, I64, I64, I64, I64, P, P, P, P]
        lib.oracle_group_acc.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P]
        lib.oracle_linear.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, P, P, P]
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_w4_code.argtypes = [P, I64]
        lib.oracle_w6_code.argtypes = [P, I64]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def decode(bits: int, canon: np.ndarray, K: int) -> np.ndarray:
    """Decoded weight codes int8[N][K] from canonical bytes."""
    canon = _c(canon, np.uint8)
    N = canon.shape[0]
    w = np.empty((N, K), np.int8)
    if _load().oracle_decode(bits, N, K, _p(canon), _p(w)):
        raise ValueError("bad bits")
    return w


def quantize_act(x_bf16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row int8 quantisation of bf16 activations: returns (q int8[M][K], s fp32[M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    _load().oracle_quantize_act(M, K, _p(x), _p(q), _p(s))
    return q, s


def rmsnorm_bf16(x_bf16: np.ndarray) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    t = np.empty((M, K), np.uint16)
    _load().oracle_rmsnorm_bf16(M, K, _p(x), _p(t))
    return t


def group_acc(bits: int, q: np.ndarray, canon: np.ndarray) -> np.ndarray:
    """int32 acc[M][N][K/128] of exact group dot products."""
    q = _c(q, np.int8)
    canon = _c(canon, np.uint8)
    M, K = q.shape
    N = canon.shape[0]
    acc = np.empty((M, N, K // GROUP), np.int32)
    if _load().oracle_group_acc(bits, M, N, K, _p(q), _p(canon), _p(acc)):
        raise ValueError("bad bits or K")
    return acc


def linear(bits: int, q: np.ndarray, s: np.ndarray, canon: np.ndarray, scales: np.ndarray,
           want_pre: bool = False):
    """bf16 y[M][N] (uint16 bit patterns); with want_pre also the fp64 value before rounding."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    canon = _c(canon, np.uint8)
    scales = _c(scales, np.float16)
    M, K = q.shape
    N = canon.shape[0]
    y = np.empty((M, N), np.uint16)
    pre = np.empty((M, N), np.float64) if want_pre else None
    rc = _load().oracle_linear(bits, M, N, K, _p(q), _p(s), _p(canon), _p(scales),
                               _p(pre) if want_pre else None, _p(y))
    if rc:
        raise ValueError("bad bits or K")
    return (y, pre) if want_pre else y


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """Run later oracle calls on n OpenMP threads (timing only; results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def f64_to_bf16(v: float) -> int:
    return int(_load().oracle_f64_to_bf16(float(v)))


def f16_to_f64(h: int) -> float:
    return float(_load().oracle_f16_to_f64(int(h)))


def wrmsnorm_bf16(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """Weighted RMSNorm of bf16 rows with bf16 per-column weights (see oracle.c)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    w = _c(w_bf16, np.uint16).reshape(-1)
    assert w.size == K
    t = np.empty((M, K), np.uint16)
    _load().oracle_wrmsnorm_bf16(M, K, _p(x), _p(w), _p(t))
    return t


def swiglu_bf16(g_bf16: np.ndarray, u_bf16: np.ndarray) -> np.ndarray:
    """h = bf16(silu(g) * u), evaluated in fp64 (see oracle.c)."""
    g = _c(g_bf16, np.uint16)
    u = _c(u_bf16, np.uint16)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.uint16)
    _load().oracle_swiglu_bf16(g.size, _p(g), _p(u), _p(h))
    return h


def decode_attention(q_bf16: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, P: int) -> np.ndarray:
    """Split-prefix decode attention of the "Paying attention to the attention!"
    section, by its definition (see oracle.c): q [M][n_q][D], caches
    [n_kv][L][D] (bf16 bits) with the M new tokens' keys and values at
    positions P .. P+M-1; token i attends to positions 0 .. P+i.  Returns bf16
    bits [M][n_q][D]."""
    q = _c(q_bf16, np.uint16)
    k = _c(k_cache, np.uint16)
    v = _c(v_cache, np.uint16)
    M, n_q, D = q.shape
    n_kv, L, D2 = k.shape
    assert D2 == D and v.shape == k.shape and n_q % n_kv == 0 and P + M <= L
    o = np.empty((M, n_q, D), np.uint16)
    rc = _load().oracle_decode_attention(M, n_q, n_kv, D, P, L, _p(q), _p(k), _p(v), _p(o))
    assert rc == 0
    return o


PRO_QUANT = 0
PRO_RMSNORM_QUANT = 1
PRO_WRMSNORM_QUANT = 2
PRO_SWIGLU_QUANT = 3


def prologue_input(x_bf16: np.ndarray, prologue: int, norm_w=None, u_bf16=None) -> np.ndarray:
    """The bf16 values a prologue hands to the quantisation."""
    if prologue == PRO_RMSNORM_QUANT:
        return rmsnorm_bf16(x_bf16)
    if prologue == PRO_WRMSNORM_QUANT:
        return wrmsnorm_bf16(x_bf16, norm_w)
    if prologue == PRO_SWIGLU_QUANT:
        return swiglu_bf16(x_bf16, u_bf16)
    return x_bf16


def prologue_quant(x_bf16: np.ndarray, prologue: int, norm_w=None, u_bf16=None):
    """The quantisation in front of a linear, with its optional prologue."""
    return quantize_act(prologue_input(x_bf16, prologue, norm_w, u_bf16))


def op(bits: int, x_bf16: np.ndarray, prologue: int, canon: np.ndarray, scales: np.ndarray,
       norm_w=None, u_bf16=None):
    q, s = prologue_quant(x_bf16, prologue, norm_w, u_bf16)
    return linear(bits, q, s, canon, scales)


def layer_sequence(bits: int, ops: list[dict], bufs: dict, weights) -> dict:
    """Run a decode-step walk op by op.

    ``ops``: dicts with K, N, in_buf, out_buf, prologue, matrix, and for the
    weighted RMSNorm ``norm_w`` (bf16 [K]), for SwiGLU ``in_buf2`` (the up
    buffer).  ``bufs``: buffer index -> bf16 array [M][width] (modified in
    place and returned).  ``weights(matrix_index) -> (canon, scales)``.  Op i
    reads columns [0, K) of its input buffer(s) and overwrites its whole
    output buffer.
    """
    for o in ops:
        x = np.ascontiguousarray(bufs[o["in_buf"]][:, : o["K"]])
        u = np.ascontiguousarray(bufs[o["in_buf2"]][:, : o["K"]]) if o["prologue"] == PRO_SWIGLU_QUANT else None
        canon, scales = weights(o["matrix"])
        bufs[o["out_buf"]] = op(bits, x, o["prologue"], canon, scales, o.get("norm_w"), u)
    return bufs
