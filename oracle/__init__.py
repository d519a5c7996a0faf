"""ctypes binding of the CPU oracle (qerl_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's CPU-baseline leg. The product
library never imports this package, and this package never imports the product library.

Arrays are numpy: bf16 tensors are uint16 bit patterns, NVFP4 and MXFP4 codes and their E4M3 and E8M0 scales are uint8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qerl_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
CXXFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", *CXXFLAGS, _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


# the same source built with AddressSanitizer and UndefinedBehaviorSanitizer (the sanitizer test loads it in a
# process started with the ASan runtime preloaded, through QERL_ORACLE_LIB)
SANITIZE_FLAGS = ["-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                  "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build_sanitized(out: str) -> str:
    subprocess.check_call(["g++", *SANITIZE_FLAGS, _SRC, "-o", out])
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("QERL_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        P, i64, i32, dbl, f32, u16, u64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                           ctypes.c_float, ctypes.c_uint16, ctypes.c_uint64)
        sig = {
            "orc_bf16_value": ([u16], dbl),
            "orc_bf16_round": ([dbl], u16),
            "orc_bf16_round_array": ([P, i64, P], None),
            "orc_e2m1_value": ([i32], dbl),
            "orc_e4m3_value": ([i32], dbl),
            "orc_e4m3_encode": ([dbl], i32),
            "orc_nvfp4_code": ([u16, dbl], i32),
            "orc_nvfp4_bytes": ([i64, i64], i64),
            "orc_nvfp4_quantize": ([P, i64, i64, i64, i32, P, P, P, P], None),
            "orc_nvfp4_quantize_rows": ([P, i64, i64, i64, P, i64, P, P, P, P], None),
            "orc_nvfp4_dequantize": ([P, P, f32, i64, i64, P, P], None),
            "orc_aqn_sigma": ([i32, dbl, dbl], dbl),
            "orc_aqn_rmsnorm": ([P, i64, i64, i64, P, P, i64, f32, f32, P, P], None),
            "orc_philox4x64_10": ([P, P, P], None),
            "orc_aqn_noise": ([u64, u64, u64, i64, i64, i64, P, i64], None),
            "orc_lora_linear": ([P, i64, i64, i64, P, P, f32, i64, P, P, i32, dbl, P], None),
            "orc_mxfp4_quantize": ([P, i64, i64, i64, P, P, P], None),
            "orc_mxfp4_dequantize": ([P, P, i64, i64, P, P], None),
            "orc_mxfp4_lora_linear": ([P, i64, i64, i64, P, P, i64, P, P, i32, dbl, P], None),
            "orc_dense_linear": ([P, i64, i64, P, i64, P], None),
            "orc_group_advantage": ([P, i32, i32, dbl, P], None),
            "orc_silu_mul": ([P, P, i64, P], None),
            "orc_grpo_surrogate": ([P, P, i64, P, P, i32, i32, dbl, dbl, i32, P, P, P], None),
            "orc_lora_linear_backward": ([P, i64, i64, P, i64, P, P, f32, P, P, i32, dbl, P, P, P], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- formats -----------------------------------------------------------------------------------------------------
def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(int(b))


def bf16_round(v: float) -> int:
    return int(lib().orc_bf16_round(float(v)))


def bf16_round_array(v: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns, one RNE rounding each."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_bf16_round_array(_p(a), a.size, _p(out))
    return out


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(int(byte))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def nvfp4_code(w_bf16: int, S: float) -> int:
    return int(lib().orc_nvfp4_code(int(w_bf16), float(S)))


def nvfp4_bytes(n: int, k: int) -> int:
    return int(lib().orc_nvfp4_bytes(n, k))


# ---- quantizer ---------------------------------------------------------------------------------------------------
def nvfp4_quantize(w: np.ndarray, scale_mode: int = 0, s_b: np.ndarray | None = None, s_g: float | None = None):
    """W bf16 [n, k] -> (codes u8 [n, k/2], s_b u8 [n, k/16], s_g float, flags int); canonical layout."""
    w = _c(w, np.uint16)
    n, k = w.shape
    assert k % 16 == 0
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    sb = np.zeros((n, k // 16), dtype=np.uint8) if s_b is None else _c(s_b, np.uint8).copy()
    sg = np.array([0.0 if s_g is None else s_g], dtype=np.float32)
    flags = np.zeros(1, dtype=np.int32)
    lib().orc_nvfp4_quantize(_p(w), n, k, k, int(scale_mode), _p(codes), _p(sb), _p(sg), _p(flags))
    return codes, sb, float(sg[0]), int(flags[0])


def nvfp4_quantize_rows(w: np.ndarray, rows) -> tuple:
    """The amax-rule quantization of the given rows of W bf16 [n, k]: s_g from the whole tensor, then block scales and
    codes of those rows only -> (codes u8 [len(rows), k/2], s_b u8 [len(rows), k/16], s_g float, flags int)."""
    w = _c(w, np.uint16)
    n, k = w.shape
    assert k % 16 == 0
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.ndim == 1 and (rows.size == 0 or (rows.min() >= 0 and rows.max() < n))
    codes = np.zeros((rows.size, k // 2), dtype=np.uint8)
    sb = np.zeros((rows.size, k // 16), dtype=np.uint8)
    sg = np.zeros(1, dtype=np.float32)
    flags = np.zeros(1, dtype=np.int32)
    lib().orc_nvfp4_quantize_rows(_p(w), n, k, k, _p(rows), rows.size, _p(codes), _p(sb), _p(sg), _p(flags))
    return codes, sb, float(sg[0]), int(flags[0])


def nvfp4_dequantize(codes: np.ndarray, s_b: np.ndarray, s_g: float):
    """-> (exact fp64 [n, k], RNE f32 [n, k])."""
    codes = _c(codes, np.uint8)
    s_b = _c(s_b, np.uint8)
    n, k2 = codes.shape
    k = 2 * k2
    we = np.empty((n, k), dtype=np.float64)
    wf = np.empty((n, k), dtype=np.float32)
    lib().orc_nvfp4_dequantize(_p(codes), _p(s_b), float(s_g), n, k, _p(we), _p(wf))
    return we, wf


# ---- AQN ---------------------------------------------------------------------------------------------------------
def aqn_sigma(stage: int, start: float = 1e-2, end: float = 5e-4) -> float:
    return float(lib().orc_aqn_sigma(int(stage), float(start), float(end)))


def aqn_rmsnorm(x: np.ndarray, gamma: np.ndarray, noise: np.ndarray | None, sigma: float, eps: float = 1e-6,
                noise_per_row: bool = False):
    """x bf16 [m, d] -> (h exact fp64 [m, d], h bf16 [m, d])."""
    x = _c(x, np.uint16)
    m, d = x.shape
    gamma = _c(gamma, np.uint16)
    nz = None if noise is None else _c(noise, np.float32)
    noise_ld = d if noise_per_row else 0
    he = np.empty((m, d), dtype=np.float64)
    hb = np.empty((m, d), dtype=np.uint16)
    lib().orc_aqn_rmsnorm(_p(x), m, d, d, _p(gamma), _p(nz), noise_ld, float(sigma), float(eps), _p(he), _p(hb))
    return he, hb


def philox4x64_10(counter, key) -> np.ndarray:
    """One Philox4x64-10 block: counter (4 words) and key (2 words) -> 4 uint64 words."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64))
    out = np.empty(4, dtype=np.uint64)
    lib().orc_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def aqn_noise(seed: int, stream: int, row_offset: int, draw_rows: int, m: int, d: int) -> np.ndarray:
    """Seeded standard-normal noise eps [m, d] f32 (Philox4x64-10 + Box-Muller; see orc_aqn_noise)."""
    out = np.empty((m, d), dtype=np.float32)
    lib().orc_aqn_noise(int(seed), int(stream), int(row_offset), int(draw_rows), m, d, _p(out), d)
    return out


# ---- linear ------------------------------------------------------------------------------------------------------
def lora_linear(h: np.ndarray, codes: np.ndarray, s_b: np.ndarray, s_g: float, A: np.ndarray | None,
                B: np.ndarray | None, lam: float) -> np.ndarray:
    """h bf16 [m, k]; NVFP4 W [n, k] canonical; A bf16 [r, k]; B bf16 [n, r] -> y fp64 [m, n]."""
    h = _c(h, np.uint16)
    m, k = h.shape
    codes = _c(codes, np.uint8)
    s_b = _c(s_b, np.uint8)
    n = codes.shape[0]
    assert codes.shape[1] * 2 == k
    r = 0
    if A is not None:
        A = _c(A, np.uint16)
        B = _c(B, np.uint16)
        r = A.shape[0]
        assert A.shape == (r, k) and B.shape == (n, r)
    y = np.empty((m, n), dtype=np.float64)
    lib().orc_lora_linear(_p(h), m, k, k, _p(codes), _p(s_b), float(s_g), n, _p(A), _p(B), r, float(lam), _p(y))
    return y


def lora_linear_backward(g: np.ndarray, h: np.ndarray, codes: np.ndarray, s_b: np.ndarray, s_g: float,
                         A: np.ndarray | None, B: np.ndarray | None, lam: float, want=("dh", "dA", "dB")):
    """Backward of lora_linear through the frozen NVFP4 weight. g bf16 [m, n] (dL/dy), h bf16 [m, k], NVFP4 W [n, k]
    canonical, A bf16 [r, k], B bf16 [n, r] -> dict of fp64 dh [m, k], dA [r, k], dB [n, r] (those in `want`)."""
    g = _c(g, np.uint16)
    h = _c(h, np.uint16)
    m, n = g.shape
    k = h.shape[1]
    assert h.shape[0] == m and codes.shape == (n, k // 2)
    r = 0
    if A is not None:
        A = _c(A, np.uint16)
        B = _c(B, np.uint16)
        r = A.shape[0]
        assert A.shape == (r, k) and B.shape == (n, r)
    out = {"dh": np.empty((m, k)) if "dh" in want else None, "dA": np.empty((r, k)) if "dA" in want else None,
           "dB": np.empty((n, r)) if "dB" in want else None}
    lib().orc_lora_linear_backward(_p(g), m, n, _p(h), k, _p(_c(codes, np.uint8)), _p(_c(s_b, np.uint8)), float(s_g),
                                   _p(A), _p(B), r, float(lam), _p(out["dh"]), _p(out["dA"]), _p(out["dB"]))
    return {key: v for key, v in out.items() if v is not None}


def mxfp4_quantize(w: np.ndarray):
    """W bf16 [n, k] (k % 32 == 0) -> (codes u8 [n, k/2], E8M0 scales u8 [n, k/32], flags int); canonical MX layout
    (OCP MX: one power-of-two scale per 32 weights, E2M1 elements)."""
    w = _c(w, np.uint16)
    n, k = w.shape
    assert k % 32 == 0
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    sc = np.zeros((n, k // 32), dtype=np.uint8)
    flags = np.zeros(1, dtype=np.int32)
    lib().orc_mxfp4_quantize(_p(w), n, k, k, _p(codes), _p(sc), _p(flags))
    return codes, sc, int(flags[0])


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray):
    """-> (exact fp64 [n, k], RNE f32 [n, k])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, k2 = codes.shape
    k = 2 * k2
    assert scales.shape == (n, k // 32)
    we = np.empty((n, k), dtype=np.float64)
    wf = np.empty((n, k), dtype=np.float32)
    lib().orc_mxfp4_dequantize(_p(codes), _p(scales), n, k, _p(we), _p(wf))
    return we, wf


def mxfp4_lora_linear(h: np.ndarray, codes: np.ndarray, scales: np.ndarray, A: np.ndarray | None,
                      B: np.ndarray | None, lam: float) -> np.ndarray:
    """h bf16 [m, k]; MXFP4 W [n, k] canonical; A bf16 [r, k]; B bf16 [n, r] -> y fp64 [m, n]."""
    h = _c(h, np.uint16)
    m, k = h.shape
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n = codes.shape[0]
    assert codes.shape[1] * 2 == k and scales.shape == (n, k // 32)
    r = 0
    if A is not None:
        A = _c(A, np.uint16)
        B = _c(B, np.uint16)
        r = A.shape[0]
        assert A.shape == (r, k) and B.shape == (n, r)
    y = np.empty((m, n), dtype=np.float64)
    lib().orc_mxfp4_lora_linear(_p(h), m, k, k, _p(codes), _p(scales), n, _p(A), _p(B), r, float(lam), _p(y))
    return y


def dense_linear(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    w = _c(w, np.uint16)
    m, k = h.shape
    n = w.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    lib().orc_dense_linear(_p(h), m, k, _p(w), n, _p(y))
    return y


def group_advantage(rewards: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """rewards f32 [groups, g] -> advantages fp64 [groups, g]."""
    R = _c(rewards, np.float32)
    groups, g = R.shape
    adv = np.empty((groups, g), dtype=np.float64)
    lib().orc_group_advantage(_p(R), groups, g, float(eps), _p(adv))
    return adv


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    g = _c(gate, np.float64)
    u = _c(up, np.float64)
    out = np.empty_like(g)
    lib().orc_silu_mul(_p(g), _p(u), g.size, _p(out))
    return out


def grpo_surrogate(logp: np.ndarray, logp_old: np.ndarray, lengths, adv, clip_low: float = 0.2,
                   clip_high: float = 0.2, agg: int = 0):
    """GRPO token ratios and clipped surrogate (see orc_grpo_surrogate). logp, logp_old f32 [n_seq, t_max];
    lengths int [n_seq]; adv f32 [n_seq] -> (surrogate fp64 [n_seq, t_max], grad fp64 [n_seq, t_max], stats dict)."""
    lp = _c(logp, np.float32)
    lo = _c(logp_old, np.float32)
    n_seq, t_max = lp.shape
    ln = _c(lengths, np.int32)
    A = _c(adv, np.float32)
    sur = np.empty((n_seq, t_max), dtype=np.float64)
    g = np.empty((n_seq, t_max), dtype=np.float64)
    st = np.empty(6, dtype=np.float64)
    lib().orc_grpo_surrogate(_p(lp), _p(lo), t_max, _p(ln), _p(A), n_seq, t_max, float(clip_low), float(clip_high),
                             int(agg), _p(sur), _p(g), _p(st))
    keys = ("loss", "ratio_mean", "ratio_min", "ratio_max", "tokens", "clipped")
    return sur, g, dict(zip(keys, st.tolist()))


# ---- decoder layer at decode (composition of the functions above) -------------------------------------------------
def gqa_broadcast(v: np.ndarray, group: int, head_dim: int) -> np.ndarray:
    """Each key/value head's vector repeated for the `group` query heads that share it (attention over a single key
    position: the output of every query head in the group is that head's value)."""
    m, kv = v.shape
    heads = kv // head_dim
    return np.repeat(v.reshape(m, heads, 1, head_dim), group, axis=2).reshape(m, kv * group)


def decoder_layer(x, q, lora, gamma1, gamma2, noise1, noise2, sigma, lam, group, head_dim, eps=1e-6):
    """Oracle of one decode layer. q[name] = (codes, s_b, s_g) canonical NVFP4; lora[name] = (A, B) bf16 or None.
    bf16 rounding happens where the device stores bf16 tensors: the norm outputs, q/k/v, x2, SiLU(g)*u, out.
    Returns a dict of the bf16 tensors (uint16 bit patterns)."""
    def lin(h, name):
        c, s, g = q[name]
        A, B = lora.get(name, (None, None))
        return lora_linear(h, c, s, g, A, B, lam)

    _, h1 = aqn_rmsnorm(x, gamma1, noise1, sigma, eps)
    qo = bf16_round_array(lin(h1, "q"))
    ko = bf16_round_array(lin(h1, "k"))
    vo = bf16_round_array(lin(h1, "v"))
    attn = gqa_broadcast(vo, group, head_dim)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x2 = bf16_round_array(lin(attn, "o") + xf)
    _, h2 = aqn_rmsnorm(x2, gamma2, noise2, sigma, eps)
    a = bf16_round_array(silu_mul(lin(h2, "gate"), lin(h2, "up")))
    x2f = (x2.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = bf16_round_array(lin(a, "down") + x2f)
    return {"q": qo, "k": ko, "attn": attn, "x2": x2, "a": a, "out": out}
