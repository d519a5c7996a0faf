"""Seeded synthetic inputs (bf16 / f32 tensors as numpy arrays) for the tests and the benchmark.

Holds no NVFP4, LoRA or AQN arithmetic: it only draws numbers and stores them in input formats. The generator is
SplitMix64 (counter-based; see synth.c for the definition) followed by Box-Muller normals.

Seeds follow one convention: base 20251013, xor (workload id << 48), xor (layer << 32), xor tensor id.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

BASE_SEED = 20251013

# tensor ids inside one decoder layer
TENSOR_IDS = {
    "w_q": 1, "w_k": 2, "w_v": 3, "w_o": 4, "w_gate": 5, "w_up": 6, "w_down": 7,
    "a_q": 11, "a_k": 12, "a_v": 13, "a_o": 14, "a_gate": 15, "a_up": 16, "a_down": 17,
    "b_q": 21, "b_k": 22, "b_v": 23, "b_o": 24, "b_gate": 25, "b_up": 26, "b_down": 27,
    "eps_norm1": 31, "eps_norm2": 32, "x": 40, "rewards": 41, "block_exp": 42, "gamma": 43,
}


def seed_for(workload: int, layer: int, tensor: str | int) -> int:
    tid = TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    return (BASE_SEED ^ (int(workload) << 48) ^ (int(layer) << 32) ^ tid) & 0xFFFFFFFFFFFFFFFF


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, dbl, ptr, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.syn_splitmix64.argtypes = [u64, u64]
        lib.syn_splitmix64.restype = u64
        lib.syn_uniform_f64.argtypes = [u64, i64, ptr]
        lib.syn_normal_f64.argtypes = [u64, i64, ptr]
        lib.syn_normal_f32.argtypes = [u64, dbl, i64, ptr]
        lib.syn_normal_bf16.argtypes = [u64, dbl, i64, ptr]
        lib.syn_student_t4_bf16.argtypes = [u64, dbl, i64, i64, u64, i32, ptr]
        lib.syn_bernoulli_f32.argtypes = [u64, dbl, i64, ptr]
        for f in ("syn_uniform_f64", "syn_normal_f64", "syn_normal_f32", "syn_normal_bf16", "syn_student_t4_bf16",
                  "syn_bernoulli_f32"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def splitmix64(seed: int, i: int) -> int:
    return int(_load().syn_splitmix64(seed, i))


def uniform(seed: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    _load().syn_uniform_f64(seed, out.size, out.ctypes.data)
    return out


def normal_f64(seed: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    _load().syn_normal_f64(seed, out.size, out.ctypes.data)
    return out


def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().syn_normal_f32(seed, float(std), out.size, out.ctypes.data)
    return out


def normal_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of std * N(0, 1)."""
    out = np.empty(shape, dtype=np.uint16)
    _load().syn_normal_bf16(seed, float(std), out.size, out.ctypes.data)
    return out


def student_t4_bf16(seed: int, shape, scale: float, block: int = 0, exp_seed: int = 0, emin: int = -14):
    out = np.empty(shape, dtype=np.uint16)
    _load().syn_student_t4_bf16(seed, float(scale), out.size, int(block), exp_seed, int(emin), out.ctypes.data)
    return out


def bernoulli_f32(seed: int, shape, p: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().syn_bernoulli_f32(seed, float(p), out.size, out.ctypes.data)
    return out


def bf16_const(value: float, shape) -> np.ndarray:
    """bf16 bit pattern of a constant that bf16 represents exactly (e.g. gamma = 1)."""
    b = np.array([value], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, "constant is not exactly representable in bf16"
    return np.full(shape, b >> 16, dtype=np.uint16)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 values (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)
