"""Seeded synthetic inputs shared by the oracle and the GPU harness.

Holds no decoder arithmetic: only the counter-based generator (SplitMix64 +
Box-Muller, bf16 round-to-nearest-even; definitions in ``synth.c``), the
workload shapes, and the recipe that says which seed and scale each weight
tensor is drawn with.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build_host()
        L = ctypes.CDLL(path)
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        L.synth_splitmix64_at.restype = u64
        L.synth_splitmix64_at.argtypes = [u64, u64]
        L.synth_tensor_seed.restype = u64
        L.synth_tensor_seed.argtypes = [u64, u32, u32]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_normal_bf16.restype = None
        L.synth_normal_bf16.argtypes = [ctypes.c_void_p, u64, u64, ctypes.c_double, u64]
        L.synth_normal_bf16_as_f32.restype = None
        L.synth_normal_bf16_as_f32.argtypes = [ctypes.c_void_p, u64, u64, ctypes.c_double, u64]
        L.synth_tokens.restype = None
        L.synth_tokens.argtypes = [ctypes.c_void_p, u64, u64, u32]
        _LIB = L
    return _LIB


def splitmix64_at(state, i):
    return lib().synth_splitmix64_at(state & (2**64 - 1), i)


def tensor_seed(base, layer, tensor_id):
    return lib().synth_tensor_seed(base, layer, tensor_id)


def normal_bf16(n, seed, sigma, offset=0):
    """bf16 bit patterns (uint16) of sigma * N(0,1) elements offset .. offset+n-1."""
    out = np.empty(int(n), dtype=np.uint16)
    if n:
        lib().synth_normal_bf16(out.ctypes.data, int(n), seed, float(sigma), int(offset))
    return out


def normal_bf16_f32(n, seed, sigma, offset=0):
    """The same values as normal_bf16, widened to fp32 (exact)."""
    out = np.empty(int(n), dtype=np.float32)
    if n:
        lib().synth_normal_bf16_as_f32(out.ctypes.data, int(n), seed, float(sigma), int(offset))
    return out


def tokens(n, seed, vocab):
    out = np.empty(int(n), dtype=np.int32)
    if n:
        lib().synth_tokens(out.ctypes.data, int(n), seed, int(vocab))
    return out


def f32_to_bf16(x):
    return int(lib().synth_f32_to_bf16(float(x)))


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16 array) to fp32, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
