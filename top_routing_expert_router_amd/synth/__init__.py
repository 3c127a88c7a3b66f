"""Seeded synthetic inputs (counter-based SplitMix64 + Box-Muller), see synth.c.

This module holds no arithmetic of the MoE method.  It is the one piece of
code that both the GPU path's callers (tests, bench, smoke) and the CPU oracle's
tests use: both sides receive the very same input bits from here.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_splitmix64.restype = u64
        L.synth_splitmix64.argtypes = [u64, u64]
        for name in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [u64, i64, i64, dbl, vp]
        L.synth_u64.restype = None
        L.synth_u64.argtypes = [u64, i64, i64, vp]
        _lib = L
    return _lib


def tensor_seed(run_id: int, j: int) -> int:
    """Seed of tensor j of run `run_id`: 1000*run + j (x=0, Wg=1, bias=2, W1=3, W3=4, W2=5)."""
    return 1000 * int(run_id) + int(j)


def splitmix64(state: int, j: int) -> int:
    return int(lib().synth_splitmix64(ctypes.c_uint64(state), ctypes.c_uint64(j)))


def normal(seed: int, count: int, sigma: float, dtype: str, first: int = 0, out=None):
    """Elements [first, first+count) of the seeded N(0, sigma^2) tensor.

    dtype: "f64" -> float64, "f32" -> float32, "bf16" -> uint16 holding bf16 bits.
    """
    npdt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[dtype]
    if out is None:
        out = np.empty(int(count), dtype=npdt)
    else:
        assert out.dtype == npdt and out.size == count and out.flags.c_contiguous
    if count:
        fn = {"f64": lib().synth_normal_f64, "f32": lib().synth_normal_f32, "bf16": lib().synth_normal_bf16}[dtype]
        fn(seed, int(first), int(count), float(sigma), out.ctypes.data)
    return out


def u64(seed: int, count: int, first: int = 0):
    out = np.empty(int(count), dtype=np.uint64)
    if count:
        lib().synth_u64(seed, int(first), int(count), out.ctypes.data)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (a bf16 is the top half of a binary32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
