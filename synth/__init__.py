"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module only draws random numbers and packs them into GGML block bytes; it
holds none of the dequant-GEMV arithmetic (no dequantisation, no dot product,
no activation), and it imports neither the oracle nor the HIP binding.

Recipes (the workload definitions that accompany the pages; the pages
themselves give no values):
  * Q8_0 weights: dense W ~ N(0, 0.02) (standard deviation 0.02) drawn in f64 and
    cast to f32, then quantised per 32-element row block: d = amax/127 in f32,
    q = round(w/d) (f32 quotient, rounded half away from zero, clamped to
    [-127, 127]), d stored as fp16 (round to nearest even), packed as 34-byte
    blocks (d little-endian, then 32 int8), row-major n_out x n_in.
    amax = 0 gives d = 0 and q = 0.
  * Q4_K weights: per 256-element super-block, d and dmin uniform on
    [1e-4, 1e-3] (f64, then fp16 RNE), 12 uniform random bytes for the packed
    scales/mins (every bit of the 12 bytes is used, so this is the same as
    uniform 6-bit scales and mins), 128 uniform random bytes of nibbles.
  * Activations and residuals: N(0, 1) drawn in f64, cast to f32.
  * Seeds: numpy default_rng (PCG64); per tensor seed = 1000*workload + index.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_ELEMS = 32
Q4K_BLOCK_BYTES = 144
Q4K_BLOCK_ELEMS = 256


def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in f64 with PCG64(seed), cast to f32."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * std).astype(np.float32)


def quantize_q8_0(w: np.ndarray) -> np.ndarray:
    """Pack a dense f32 (n_out, n_in) matrix into GGML Q8_0 bytes (uint8, flat)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n_out, n_in = w.shape
    assert n_in % Q8_0_BLOCK_ELEMS == 0
    nb = n_in // Q8_0_BLOCK_ELEMS
    blocks = w.reshape(n_out, nb, Q8_0_BLOCK_ELEMS)
    amax = np.max(np.abs(blocks), axis=2)                      # f32
    d = (amax / np.float32(127.0)).astype(np.float32)          # f32 quotient
    safe = np.where(d == 0, np.float32(1.0), d).astype(np.float32)
    v = (blocks / safe[:, :, None]).astype(np.float32)         # f32 quotient
    v64 = v.astype(np.float64)
    q = np.trunc(v64 + np.copysign(0.5, v64))                  # half away from zero
    q = np.clip(q, -127, 127)
    q[d == 0] = 0
    out = np.empty((n_out, nb, Q8_0_BLOCK_BYTES), np.uint8)
    out[:, :, 0:2] = d.astype(np.float16).view(np.uint8).reshape(n_out, nb, 2)
    out[:, :, 2:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(-1)


def q8_0_weights(seed: int, n_out: int, n_in: int, std: float = 0.02):
    """(packed Q8_0 bytes, the dense f32 matrix they were quantised from)."""
    w = normal_f32(seed, (n_out, n_in), std)
    return quantize_q8_0(w), w


def q4k_weights(seed: int, n_out: int, n_in: int, lo: float = 1e-4, hi: float = 1e-3) -> np.ndarray:
    """Random GGML Q4_K bytes (uint8, flat), row-major n_out x n_in."""
    assert n_in % Q4K_BLOCK_ELEMS == 0
    nsb = n_in // Q4K_BLOCK_ELEMS
    rng = np.random.default_rng(seed)
    blk = np.empty((n_out, nsb, Q4K_BLOCK_BYTES), np.uint8)
    d = rng.uniform(lo, hi, (n_out, nsb)).astype(np.float16)
    dmin = rng.uniform(lo, hi, (n_out, nsb)).astype(np.float16)
    blk[:, :, 0:2] = d.view(np.uint8).reshape(n_out, nsb, 2)
    blk[:, :, 2:4] = dmin.view(np.uint8).reshape(n_out, nsb, 2)
    blk[:, :, 4:] = rng.integers(0, 256, (n_out, nsb, Q4K_BLOCK_BYTES - 4), dtype=np.uint8)
    return blk.reshape(-1)


Q6K_BLOCK_BYTES, Q6K_BLOCK_ELEMS = 210, 256


def q6k_weights(seed: int, n_out: int, n_in: int, lo: float = 1e-4, hi: float = 1e-3) -> np.ndarray:
    """Random GGML Q6_K bytes (uint8, flat), row-major n_out x n_in: random
    quant bytes, int8 scales in [-64, 63], fp16 d in [lo, hi]."""
    assert n_in % Q6K_BLOCK_ELEMS == 0
    nsb = n_in // Q6K_BLOCK_ELEMS
    rng = np.random.default_rng(seed)
    blk = np.empty((n_out, nsb, Q6K_BLOCK_BYTES), np.uint8)
    blk[:, :, 0:192] = rng.integers(0, 256, (n_out, nsb, 192), dtype=np.uint8)
    blk[:, :, 192:208] = rng.integers(-64, 64, (n_out, nsb, 16)).astype(np.int8).view(np.uint8)
    d = rng.uniform(lo, hi, (n_out, nsb)).astype(np.float16)
    blk[:, :, 208:210] = d.view(np.uint8).reshape(n_out, nsb, 2)
    return blk.reshape(-1)


def fnv1a64_py(raw: bytes | np.ndarray, n_in: int, n_out: int) -> int:
    """Content fingerprint for run logs: FNV-1a over the bytes, then n_in and
    n_out each folded in as a whole 64-bit word (the pages' weight_fingerprint
    in the rustdoc source view of weight_cache.rs).  One multiply per byte in
    Python: the statement of the hash that pins the compiled fnv1a64."""
    data = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)
    mask = (1 << 64) - 1
    prime = 0x100000001B3
    h = 0xCBF29CE484222325
    for byte in data.tobytes():
        h = ((h ^ byte) * prime) & mask
    h = ((h ^ (n_in & mask)) * prime) & mask
    h = ((h ^ (n_out & mask)) * prime) & mask
    return h


_FNV_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fnv1a.c")
_FNV_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynthfnv.so")
_fnv = None


def build_fnv(force: bool = False) -> str:
    """Compile fnv1a.c with gcc (in-tree, next to this file)."""
    if force or not os.path.exists(_FNV_LIB) or os.path.getmtime(_FNV_LIB) < os.path.getmtime(_FNV_SRC):
        tmp = _FNV_LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-o", tmp, _FNV_SRC], check=True)
        os.replace(tmp, _FNV_LIB)
    return _FNV_LIB


def fnv1a64(raw: bytes | np.ndarray, n_in: int, n_out: int) -> int:
    """The same fingerprint as fnv1a64_py, computed by the compiled fnv1a.c
    (tensors of tens of MB in the benchmark logs)."""
    global _fnv
    if _fnv is None:
        lib = ctypes.CDLL(build_fnv())
        lib.synth_fnv1a64.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_fnv1a64.restype = ctypes.c_uint64
        _fnv = lib
    data = np.ascontiguousarray(np.ascontiguousarray(raw).view(np.uint8).reshape(-1))
    return int(_fnv.synth_fnv1a64(data.ctypes.data_as(ctypes.c_void_p), data.size, n_in & ((1 << 64) - 1),
                                  n_out & ((1 << 64) - 1)))


def seed(workload: int, index: int) -> int:
    return 1000 * workload + index
