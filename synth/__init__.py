"""Seeded synthetic inputs for the Medusa decode step.

This package produces the numbers every test, the smoke check and the bench
feed to both the CPU oracle and the GPU library; it computes nothing of the
decode step itself. Tensors are drawn from a Philox4x32-10 counter generator
(``synth.c``), one stream per tensor, so both sides read identical bytes.

bf16 tensors are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``libsynth.so`` in place with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, u64, u32, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
        L.syn_normal_f32.argtypes = [u64, u32, i64, i64, dbl, vp]
        L.syn_normal_bf16.argtypes = [u64, u32, i64, i64, dbl, vp]
        L.syn_u32.argtypes = [u64, u32, i64, i64, vp]
        L.syn_philox4x32_10.argtypes = [vp, vp, vp]
        for f in (L.syn_normal_f32, L.syn_normal_bf16, L.syn_u32, L.syn_philox4x32_10):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().syn_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal(seed: int, stream: int, shape, std: float, dtype: str, first: int = 0) -> np.ndarray:
    """N(0, std^2) draws; dtype 'f32' -> float32, 'bf16' -> uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib().syn_normal_f32(seed, stream, first, n, float(std), _ptr(out))
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib().syn_normal_bf16(seed, stream, first, n, float(std), _ptr(out))
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def u32(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().syn_u32(seed, stream, first, n, _ptr(out))
    return out


def uniform01(seed: int, stream: int, n: int) -> np.ndarray:
    """Doubles in the open interval (0, 1), one per 32-bit word."""
    return (u32(seed, stream, n).astype(np.float64) + 0.5) / 4294967296.0


def randint(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive (64-bit multiply-shift of a 32-bit word)."""
    w = u32(seed, stream, n).astype(np.uint64)
    span = np.uint64(hi - lo + 1)
    return (lo + ((w * span) >> np.uint64(32)).astype(np.int64)).astype(np.int32)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)
