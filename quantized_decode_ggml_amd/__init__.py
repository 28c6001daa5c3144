"""Python binding of libqdec (include/qdec.h): block-quantized dequant-GEMV/GEMM
for AMD MI355X (gfx950).

Argument marshalling only.  Every function takes torch tensors that live on the
GPU, passes their device pointers and the current HIP stream to the C ABI of the
same name, and raises QdecError on a non-zero status.  All arithmetic runs in
the library's HIP kernels; there is no CPU path.  Weights passed to the
library stay allocated until ``release`` or ``clear_cache`` (see ``_track``).
The library must have been
built (``python quantized_decode_ggml_amd/_build.py`` or
``__graft_entry__.build()``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqdec.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "qdec.h")

QDEC_OK, QDEC_EINVAL, QDEC_ENOMEM, QDEC_EHIP, QDEC_EUNSUPPORTED = 0, -1, -2, -3, -4
TYPE_F32, TYPE_Q8_0, TYPE_Q4_K, TYPE_Q6_K = 0, 8, 12, 14
GEMV_MAX_BATCH = 8
TOPK_MAX = 256

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python quantized_decode_ggml_amd/_build.py)")

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int64
_SIGS = {
    "q8_0_gemv": [_P, _I, _I, _I, _P, _P, _P],
    "q8_0_gemv_residual": [_P, _I, _I, _I, _P, _P, _P, _P],
    "q8_0_qkv": [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P],
    "q8_0_swiglu": [_P, _P, _I, _I, _I, _P, _P, _P],
    "q4k_gemv": [_P, _I, _I, _I, _P, _P, _P],
    "q6k_gemv": [_P, _I, _I, _I, _P, _P, _P],
    "qdec_rope_kv_append": [_P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _I, _P],
    "qdec_attention_decode": [_P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P],
    "q6k_dequantize": [_P, _I, _I, _P, _P],
    "q8_0_gemv_topk": [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P],
    "q8_0_gemv_topk_noalloc": [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P],
    "qdec_rmsnorm": [_P, _I, _I, _P, ctypes.c_float, _P, _P],
    "q8_0_rmsnorm_qkv": [_P, _P, _P, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P],
    "q8_0_attn_out_ffn": [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, ctypes.c_float, _P, _P],
    "q8_0_gemm_batched": [_P, _I, _I, _I, _P, _P, _P],
    "f32_gemm_batched": [_P, _I, _I, _I, _P, _P, _P],
    "qdec_prepare": [_P, ctypes.c_int, _I, _I, _P],
    "qdec_release": [_P],
    "q8_0_dequantize": [_P, _I, _I, _P, _P],
    "q4k_dequantize": [_P, _I, _I, _P, _P],
    "qdec_empty_kernel": [_P],
    "qdec_copy": [_P, _P, _I, _P],
    "qdec_stream_read": [_P, _I, ctypes.c_int, _P, _P],
    "qdec_check_plans": [_I, _I, _I],
}
for _name, _args in _SIGS.items():
    getattr(lib, _name).argtypes = _args
    getattr(lib, _name).restype = ctypes.c_int
lib.qdec_clear_cache.argtypes = []
lib.qdec_clear_cache.restype = None
lib.qdec_cache_len.argtypes = []
lib.qdec_cache_len.restype = ctypes.c_int64
lib.qdec_last_error.argtypes = []
lib.qdec_last_error.restype = ctypes.c_char_p
lib.qdec_launch_count.argtypes = []
lib.qdec_launch_count.restype = ctypes.c_uint64


class QdecError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qdec status {status}: {msg}")
        self.status = status


def declared_functions() -> list[str]:
    """Names of the functions include/qdec.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return re.findall(r"^QDEC_API\s+[\w\s\*]+?\b(\w+)\s*\(", text, re.M)


def _check(status: int):
    if status != QDEC_OK:
        raise QdecError(status, lib.qdec_last_error().decode(errors="replace"))


# The library caches a repacked copy per weight pointer and trusts the caller to
# release it before the bytes behind the pointer change.  Torch frees and reuses
# device addresses, so the binding keeps the storage of every weight it has
# passed to the library alive until release() or clear_cache(): its address
# cannot be handed to another tensor while a copy made from it exists, and a
# captured graph that reads the copy stays valid however the caller's tensor
# objects and views come and go.  Nothing is freed from a garbage-collection
# callback (which could run in the middle of a stream capture).
_pinned: dict[int, object] = {}


def _track(*weights):
    """After a successful call: keep each weight's storage alive while the
    library may hold a copy made from it."""
    for t in weights:
        if t is None or isinstance(t, int):
            continue
        ptr = t.data_ptr()
        if ptr not in _pinned:
            _pinned[ptr] = t.untyped_storage()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _batch(x: torch.Tensor, n_in: int) -> int:
    if x.numel() % n_in:
        raise ValueError(f"x has {x.numel()} elements, not a multiple of n_in={n_in}")
    return x.numel() // n_in


def _f32_out(out, batch, n, like):
    if out is None:
        out = torch.empty((batch, n), dtype=torch.float32, device=like.device)
    return out


def q8_0_gemv(w, n_in, n_out, x, out=None, stream=None):
    """out[b, i] = sum_j deq(W)[i, j] x[b, j]; w holds raw GGML Q8_0 bytes."""
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.q8_0_gemv(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(out), _stream(stream)))
    _track(w)
    return out


def q8_0_gemv_residual(w, n_in, n_out, x, residual, out=None, stream=None):
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.q8_0_gemv_residual(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(residual), _ptr(out),
                                  _stream(stream)))
    _track(w)
    return out


def q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x, q_out=None, k_out=None, v_out=None, stream=None):
    batch = _batch(x, n_in)
    q_out = _f32_out(q_out, batch, n_q, x)
    k_out = _f32_out(k_out, batch, n_kv, x)
    v_out = _f32_out(v_out, batch, n_kv, x)
    _check(lib.q8_0_qkv(_ptr(wq), _ptr(wk), _ptr(wv), n_in, n_q, n_kv, batch, _ptr(x), _ptr(q_out),
                        _ptr(k_out), _ptr(v_out), _stream(stream)))
    _track(wq, wk, wv)
    return q_out, k_out, v_out


def q8_0_swiglu(w_gate, w_up, n_in, n_out, x, out=None, stream=None):
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.q8_0_swiglu(_ptr(w_gate), _ptr(w_up), n_in, n_out, batch, _ptr(x), _ptr(out),
                           _stream(stream)))
    _track(w_gate, w_up)
    return out


def q8_0_gemv_topk(w, n_in, n_out, x, k, logits=None, top_idx=None, top_val=None, stream=None):
    """Vocabulary projection plus on-device top-k: returns (top_idx int32
    (batch, k), top_val f32 (batch, k), logits f32 (batch, n_out))."""
    batch = _batch(x, n_in)
    logits = _f32_out(logits, batch, n_out, x)
    if top_idx is None:
        top_idx = torch.empty((batch, k), dtype=torch.int32, device=x.device)
    top_val = _f32_out(top_val, batch, k, x)
    _check(lib.q8_0_gemv_topk(_ptr(w), n_in, n_out, batch, _ptr(x), k, _ptr(logits), _ptr(top_idx),
                              _ptr(top_val), _stream(stream)))
    _track(w)
    return top_idx, top_val, logits


def q8_0_gemv_topk_noalloc(w, n_in, n_out, x, k, logits, top_idx, top_val, stream=None):
    """q8_0_gemv_topk without any device allocation: w must be prepared, and the
    outputs are the caller's (no tensor is created here)."""
    batch = _batch(x, n_in)
    _check(lib.q8_0_gemv_topk_noalloc(_ptr(w), n_in, n_out, batch, _ptr(x), k, _ptr(logits), _ptr(top_idx),
                                      _ptr(top_val), _stream(stream)))
    return top_idx, top_val, logits


def rmsnorm(x, w, eps, out=None, stream=None):
    """out = x / sqrt(mean(x^2) + eps) * w per row; out may be x (in place)."""
    n = w.numel()
    batch = _batch(x, n)
    out = _f32_out(out, batch, n, x)
    _check(lib.qdec_rmsnorm(_ptr(x), n, batch, _ptr(w), float(eps), _ptr(out), _stream(stream)))
    return out


def q8_0_rmsnorm_qkv(wq, wk, wv, n_in, n_q, n_kv, h, norm_w, eps, q_out=None, k_out=None, v_out=None,
                     scratch=None, stream=None):
    """(q, k, v) = QKV(RMSNorm(h)); scratch (batch x n_in) is made when the
    norm cannot be folded (several batch rows) and none is given."""
    batch = _batch(h, n_in)
    q_out = _f32_out(q_out, batch, n_q, h)
    k_out = _f32_out(k_out, batch, n_kv, h)
    v_out = _f32_out(v_out, batch, n_kv, h)
    if scratch is None and batch > 1:
        scratch = torch.empty((batch, n_in), dtype=torch.float32, device=h.device)
    _check(lib.q8_0_rmsnorm_qkv(_ptr(wq), _ptr(wk), _ptr(wv), n_in, n_q, n_kv, batch, _ptr(h), _ptr(norm_w),
                                float(eps), _ptr(q_out), _ptr(k_out), _ptr(v_out), _ptr(scratch),
                                _stream(stream)))
    _track(wq, wk, wv)
    return q_out, k_out, v_out


def q8_0_attn_out_ffn(wo, w_gate, w_up, w_down, n_embd, n_q, n_ff, h, attn, ffn_norm, eps, scratch=None,
                      stream=None):
    """h += Wo attn; h += Wd SwiGLU(RMSNorm(h)), in place; returns h."""
    batch = _batch(h, n_embd)
    if scratch is None:
        scratch = torch.empty((batch, n_ff + n_embd), dtype=torch.float32, device=h.device)
    _check(lib.q8_0_attn_out_ffn(_ptr(wo), _ptr(w_gate), _ptr(w_up), _ptr(w_down), n_embd, n_q, n_ff, batch,
                                 _ptr(h), _ptr(attn), _ptr(ffn_norm), float(eps), _ptr(scratch),
                                 _stream(stream)))
    _track(wo, w_gate, w_up, w_down)
    return h


def q4k_gemv(w, n_in, n_out, x, out=None, stream=None):
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.q4k_gemv(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(out), _stream(stream)))
    _track(w)
    return out


def q6k_gemv(w, n_in, n_out, x, out=None, stream=None):
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.q6k_gemv(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(out), _stream(stream)))
    _track(w)
    return out


def rope_kv_append(q, k, v, pos, base, k_cache, v_cache, stream=None):
    """RoPE on q (n_head, d) and k (n_kv, d) in place for position pos, then
    k and v written at pos of the caches (n_kv, max_seq, d)."""
    n_head, d = q.shape
    n_kv, max_seq, _ = k_cache.shape
    _check(lib.qdec_rope_kv_append(_ptr(q), _ptr(k), _ptr(v), n_head, n_kv, d, int(pos), float(base), _ptr(k_cache),
                                   _ptr(v_cache), max_seq, _stream(stream)))
    return q, k


def attention_decode(q, k_cache, v_cache, n_ctx, scale, out=None, stream=None):
    """GQA softmax attention of q (n_head, d) over positions < n_ctx."""
    n_head, d = q.shape
    n_kv, max_seq, _ = k_cache.shape
    if out is None:
        out = torch.empty((n_head, d), dtype=torch.float32, device=q.device)
    _check(lib.qdec_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), n_head, n_kv, d, int(n_ctx), max_seq,
                                     float(scale), _ptr(out), _stream(stream)))
    return out


def q8_0_gemm_batched(w, n_in, n_out, x, out=None, stream=None):
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.q8_0_gemm_batched(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(out), _stream(stream)))
    _track(w)
    return out


def f32_gemm_batched(w, n_in, n_out, x, out=None, stream=None):
    batch = _batch(x, n_in)
    out = _f32_out(out, batch, n_out, x)
    _check(lib.f32_gemm_batched(_ptr(w), n_in, n_out, batch, _ptr(x), _ptr(out), _stream(stream)))
    return out


def prepare(w, qtype, n_in, n_out, stream=None):
    _check(lib.qdec_prepare(_ptr(w), int(qtype), n_in, n_out, _stream(stream)))
    _track(w)


def release(w):
    """Free the library's copies of w (graphs captured from calls on w must
    not be replayed afterwards) and stop keeping its storage alive."""
    ptr = _ptr(w)
    try:
        _check(lib.qdec_release(ptr))
    finally:
        _pinned.pop(ptr, None)


def clear_cache():
    """Free every copy and workspace (invalidates every captured graph that
    used the library) and every storage the binding kept alive."""
    lib.qdec_clear_cache()
    _pinned.clear()


def check_plans(n_in, n_out, batch):
    """Host-side extent check of every launch plan for this shape (no device
    needed); raises QdecError naming the overrun if a plan would leave its
    buffers."""
    _check(lib.qdec_check_plans(n_in, n_out, batch))


def cache_len() -> int:
    return int(lib.qdec_cache_len())


def q8_0_dequantize(w, n_in, n_out, out=None, stream=None):
    if out is None:
        out = torch.empty((n_out, n_in), dtype=torch.float32, device=w.device)
    _check(lib.q8_0_dequantize(_ptr(w), n_in, n_out, _ptr(out), _stream(stream)))
    _track(w)
    return out


def q4k_dequantize(w, n_in, n_out, out=None, stream=None):
    if out is None:
        out = torch.empty((n_out, n_in), dtype=torch.float32, device=w.device)
    _check(lib.q4k_dequantize(_ptr(w), n_in, n_out, _ptr(out), _stream(stream)))
    _track(w)
    return out


def q6k_dequantize(w, n_in, n_out, out=None, stream=None):
    if out is None:
        out = torch.empty((n_out, n_in), dtype=torch.float32, device=w.device)
    _check(lib.q6k_dequantize(_ptr(w), n_in, n_out, _ptr(out), _stream(stream)))
    _track(w)
    return out


def launch_count() -> int:
    return int(lib.qdec_launch_count())


def last_error() -> str:
    return lib.qdec_last_error().decode(errors="replace")


def empty_kernel(stream=None):
    _check(lib.qdec_empty_kernel(_stream(stream)))


def copy(dst, src, nbytes, stream=None):
    _check(lib.qdec_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def stream_read(src, nbytes, loads_per_lane, sink, stream=None):
    """Plain streaming read of nbytes of src (the HBM read ceiling probe)."""
    _check(lib.qdec_stream_read(_ptr(src), nbytes, int(loads_per_lane), _ptr(sink), _stream(stream)))
