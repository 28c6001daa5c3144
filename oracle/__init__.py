"""CPU oracle for the block-quantized dequant-GEMV/GEMM (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library and
its binding in ``quantized_decode_ggml_amd``) never does, and this package never
imports that one.

What each function computes, and which passage of the pages it follows, is
stated in ``oracle.c`` beside the C function.  Outputs of dot products are f64;
each also returns S = sum_j |w_ij x_j| (f64), the scale of the tolerances.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # QDEC_ORACLE_LIB lets the mutation tests load a deliberately broken
            # copy of the oracle to show that the pins reject it.
            path = os.environ.get("QDEC_ORACLE_LIB") or build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            lib.oracle_fp16_to_f32.argtypes = [ctypes.c_uint16]
            lib.oracle_fp16_to_f32.restype = ctypes.c_float
            lib.oracle_fp16_to_f32_array.argtypes = [P, I, P]
            lib.oracle_q4k_unpack_scales.argtypes = [P, P, P]
            lib.oracle_q8_0_dequantize.argtypes = [P, I, I, P]
            lib.oracle_q4k_dequantize.argtypes = [P, I, I, P]
            lib.oracle_q6k_dequantize.argtypes = [P, I, I, P]
            for name in ("oracle_q8_0_gemv", "oracle_q4k_gemv", "oracle_q6k_gemv", "oracle_f32_gemm"):
                getattr(lib, name).argtypes = [P, I, I, I, P, P, P]
                getattr(lib, name).restype = ctypes.c_int
            lib.oracle_q8_0_gemv_residual.argtypes = [P, I, I, I, P, P, P, P]
            lib.oracle_q8_0_gemv_residual.restype = ctypes.c_int
            lib.oracle_q8_0_qkv.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, P, P]
            lib.oracle_q8_0_qkv.restype = ctypes.c_int
            lib.oracle_q8_0_swiglu.argtypes = [P, P, I, I, I, P, P, P, P, P, P]
            lib.oracle_q8_0_swiglu.restype = ctypes.c_int
            lib.oracle_silu.argtypes = [ctypes.c_double]
            lib.oracle_silu.restype = ctypes.c_double
            lib.oracle_topk.argtypes = [P, I, I, I, P, P]
            lib.oracle_topk.restype = ctypes.c_int
            lib.oracle_rmsnorm.argtypes = [P, I, I, P, ctypes.c_double, P]
            lib.oracle_rmsnorm.restype = ctypes.c_int
            lib.oracle_rope.argtypes = [P, I, I, I, ctypes.c_double]
            lib.oracle_rope.restype = None
            lib.oracle_attention.argtypes = [P, P, P, I, I, I, I, I, ctypes.c_double, P, P]
            lib.oracle_attention.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        a = a.view(np.uint8)
    return a.reshape(-1)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int, name: str):
    if rc != 0:
        raise MemoryError(f"{name}: allocation failed")


def fp16_to_f32(h) -> np.ndarray:
    """Decode binary16 bit patterns (uint16 array) to f32 per IEEE 754."""
    h = np.ascontiguousarray(h, dtype=np.uint16).reshape(-1)
    out = np.empty(h.size, dtype=np.float32)
    _load().oracle_fp16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


def q4k_unpack_scales(s12) -> tuple[np.ndarray, np.ndarray]:
    """Unpack 12 bytes into (sc[8], m[8]) 6-bit values."""
    s = _u8(np.asarray(s12, dtype=np.uint8))
    assert s.size == 12
    sc = np.zeros(8, np.uint8)
    m = np.zeros(8, np.uint8)
    _load().oracle_q4k_unpack_scales(_ptr(s), _ptr(sc), _ptr(m))
    return sc, m


def q8_0_dequantize(w, n_in: int, n_out: int) -> np.ndarray:
    w = _u8(w)
    assert n_in % 32 == 0 and w.size >= n_out * (n_in // 32) * 34
    out = np.empty((n_out, n_in), np.float32)
    _load().oracle_q8_0_dequantize(_ptr(w), n_in, n_out, _ptr(out))
    return out


def q4k_dequantize(w, n_in: int, n_out: int) -> np.ndarray:
    w = _u8(w)
    assert n_in % 256 == 0 and w.size >= n_out * (n_in // 256) * 144
    out = np.empty((n_out, n_in), np.float32)
    _load().oracle_q4k_dequantize(_ptr(w), n_in, n_out, _ptr(out))
    return out


def _gemv(fn, w, n_in, n_out, x, wconv):
    x = _f32(x)
    batch = x.size // n_in
    assert x.size == batch * n_in and batch >= 1
    w = wconv(w)
    out = np.empty((batch, n_out), np.float64)
    s = np.empty((batch, n_out), np.float64)
    _check(fn(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(out), _ptr(s)), fn.__name__)
    return out, s


def q8_0_gemv(w, n_in: int, n_out: int, x):
    """(out, S), both (batch, n_out) f64; x is (batch, n_in) f32."""
    return _gemv(_load().oracle_q8_0_gemv, w, n_in, n_out, x, _u8)


def q4k_gemv(w, n_in: int, n_out: int, x):
    return _gemv(_load().oracle_q4k_gemv, w, n_in, n_out, x, _u8)


def q6k_dequantize(w, n_in: int, n_out: int) -> np.ndarray:
    """(n_out, n_in) f32 from raw GGML Q6_K bytes (210-byte super-blocks)."""
    w = _u8(w)
    assert n_in % 256 == 0 and w.size == n_out * (n_in // 256) * 210
    out = np.empty((n_out, n_in), np.float32)
    _load().oracle_q6k_dequantize(_ptr(w), n_in, n_out, _ptr(out))
    return out


def q6k_gemv(w, n_in: int, n_out: int, x):
    return _gemv(_load().oracle_q6k_gemv, w, n_in, n_out, x, _u8)


def f32_gemm(w, n_in: int, n_out: int, x):
    return _gemv(_load().oracle_f32_gemm, w, n_in, n_out, x, lambda a: _f32(a).reshape(-1))


def q8_0_gemv_residual(w, n_in: int, n_out: int, x, residual):
    x = _f32(x)
    batch = x.size // n_in
    r = _f32(residual).reshape(-1)
    assert r.size == batch * n_out
    w = _u8(w)
    out = np.empty((batch, n_out), np.float64)
    s = np.empty((batch, n_out), np.float64)
    _check(_load().oracle_q8_0_gemv_residual(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(r),
                                             _ptr(out), _ptr(s)), "residual")
    return out, s


def q8_0_qkv(wq, wk, wv, n_in: int, n_q: int, n_kv: int, x):
    """((q, k, v), (Sq, Sk, Sv)), each (batch, rows) f64."""
    x = _f32(x)
    batch = x.size // n_in
    outs = [np.empty((batch, n), np.float64) for n in (n_q, n_kv, n_kv)]
    ss = [np.empty((batch, n), np.float64) for n in (n_q, n_kv, n_kv)]
    _check(_load().oracle_q8_0_qkv(_ptr(_u8(wq)), _ptr(_u8(wk)), _ptr(_u8(wv)), n_in, n_q, n_kv,
                                   batch, _ptr(x), *[_ptr(o) for o in outs],
                                   *[_ptr(s) for s in ss]), "qkv")
    return tuple(outs), tuple(ss)


def q8_0_swiglu(w_gate, w_up, n_in: int, n_out: int, x):
    """dict with out, g, u, Sg, Su, each (batch, n_out) f64."""
    x = _f32(x)
    batch = x.size // n_in
    r = {k: np.empty((batch, n_out), np.float64) for k in ("out", "g", "u", "Sg", "Su")}
    _check(_load().oracle_q8_0_swiglu(_ptr(_u8(w_gate)), _ptr(_u8(w_up)), n_in, n_out, batch,
                                      _ptr(x), _ptr(r["out"]), _ptr(r["g"]), _ptr(r["u"]),
                                      _ptr(r["Sg"]), _ptr(r["Su"])), "swiglu")
    return r


def silu(z: float) -> float:
    return _load().oracle_silu(float(z))


def topk(values, k: int):
    """(idx int32, val f32), each (batch, k): the k largest values of each row,
    largest first, equal values by smaller index.  values is (batch, n) f32."""
    v = _f32(values)
    v2 = v.reshape(-1, v.shape[-1]) if v.ndim > 1 else v.reshape(1, -1)
    batch, n = v2.shape
    idx = np.empty((batch, k), np.int32)
    val = np.empty((batch, k), np.float32)
    if _load().oracle_topk(_ptr(np.ascontiguousarray(v2)), n, batch, k, _ptr(idx), _ptr(val)) != 0:
        raise ValueError(f"topk: k={k} outside [1, n={n}], or a NaN value")
    return idx, val


def rmsnorm(x, w, eps: float) -> np.ndarray:
    """f64 (batch, n): x / sqrt(mean(x^2) + eps) * w per row (oracle.c)."""
    wv = _f32(w).reshape(-1)
    n = wv.size
    xv = _f32(x).reshape(-1)
    batch = xv.size // n
    assert xv.size == batch * n and batch >= 1
    out = np.empty((batch, n), np.float64)
    if _load().oracle_rmsnorm(_ptr(xv), n, batch, _ptr(wv), float(eps), _ptr(out)) != 0:
        raise ValueError("rmsnorm: bad arguments")
    return out


def q8_0_gemv_f64(w, n_in: int, n_out: int, y) -> tuple[np.ndarray, np.ndarray]:
    """(out, S) for an f64 input y (batch, n_in), e.g. a normalised vector that
    never exists in f32: out = deq(W) y and S = |deq(W)| |y|, with deq from
    q8_0_dequantize (exact f32) and numpy's f64 matrix product as the step."""
    y = np.asarray(y, np.float64).reshape(-1, n_in)
    deq = q8_0_dequantize(w, n_in, n_out).astype(np.float64)
    return y @ deq.T, np.abs(y) @ np.abs(deq).T


def f32_gemm_f64(w, n_in: int, n_out: int, y) -> tuple[np.ndarray, np.ndarray]:
    """(out, S) of the dense batched product of ``f32_gemm`` for large shapes:
    out = y W^T and S = |y| |W|^T with W the f32 row-major (n_out, n_in)
    weights widened to f64 (exact) and numpy's f64 matrix product as the step
    (weight_cache.rs source view, try_cuda_batch_gemv: C = A B with A the
    batch x n_in hidden rows and B the transposed weight)."""
    y = np.asarray(y, np.float64).reshape(-1, n_in)
    wd = np.asarray(w, np.float32).reshape(n_out, n_in).astype(np.float64)
    return y @ wd.T, np.abs(y) @ np.abs(wd).T


def q8_0_swiglu_f64(w_gate, w_up, n_in: int, n_out: int, y) -> dict:
    """As q8_0_swiglu for an f64 input y: dict with out, g, u, Sg, Su."""
    g, sg = q8_0_gemv_f64(w_gate, n_in, n_out, y)
    u, su = q8_0_gemv_f64(w_up, n_in, n_out, y)
    silu_g = g / (1.0 + np.exp(-g))          # silu(z) = z / (1 + e^-z), as oracle_silu
    return {"out": silu_g * u, "g": g, "u": u, "Sg": sg, "Su": su}


def rope(x, pos: int, base: float) -> np.ndarray:
    """f64 (n_heads, d): adjacent pairs of each head rotated by pos * base^(-2i/d)."""
    v = np.array(x, np.float64, copy=True)
    n_heads, d = v.shape
    _load().oracle_rope(_ptr(v), n_heads, d, int(pos), float(base))
    return v


def attention(q, k_cache, v_cache, n_ctx: int, scale: float):
    """(out, A), each f64 (n_head, d): GQA softmax attention of q (n_head, d,
    any float) over positions < n_ctx of the f32 caches (n_kv, max_seq, d);
    A = sum_t p_t |V[t]| per element."""
    qv = np.ascontiguousarray(q, np.float64)
    kc = np.ascontiguousarray(k_cache, np.float32)
    vc = np.ascontiguousarray(v_cache, np.float32)
    n_head, d = qv.shape
    n_kv, max_seq, _ = kc.shape
    out = np.empty((n_head, d), np.float64)
    a = np.empty((n_head, d), np.float64)
    if _load().oracle_attention(_ptr(qv), _ptr(kc), _ptr(vc), n_head, n_kv, d, int(n_ctx), max_seq, float(scale),
                                _ptr(out), _ptr(a)) != 0:
        raise ValueError("attention: bad arguments")
    return out, a
