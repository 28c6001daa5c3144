"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded
bytes and activations.

Bars: dequantised weights bit-exact (compared as uint32); f32 paths
|gpu - oracle| <= 1e-5 * S + 1e-6 with S = sum_j |w_ij x_bj| from the oracle;
the bf16-MFMA batched GEMM <= 5e-3 * S; SwiGLU with the first-order propagated
bound (helpers.swiglu_tol).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_REL, check_f32, f32_bits, q8_weights, swiglu_tol, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_decode_ggml_amd as q
    return q


@pytest.fixture(autouse=True)
def fresh_cache(qd):
    """The repack cache is keyed by device pointer and the caller promises the
    bytes behind a cached pointer do not change until it is released.  Tests
    free and reallocate weights through torch's caching allocator, which hands
    the same addresses back, so every test starts and ends with an empty cache."""
    qd.clear_cache()
    yield
    qd.clear_cache()


def dev(a):
    return to_dev(a, torch)


def sync():
    torch.cuda.synchronize()


def host(t):
    sync()
    return t.cpu().numpy()


# -------------------------------------------------------------- dequant --

@pytest.mark.parametrize("n_out,n_in", [(1, 32), (7, 96), (256, 512), (33, 3072)])
def test_q8_0_dequant_bitexact(qd, n_out, n_in):
    raw = q8_weights(11 + n_in, n_out, n_in)
    got = host(qd.q8_0_dequantize(dev(raw), n_in, n_out))
    ref = oracle.q8_0_dequantize(raw, n_in, n_out)
    assert np.array_equal(f32_bits(got), f32_bits(ref))


def test_q8_0_dequant_bitexact_all_scales(qd):
    """Every finite fp16 d (including subnormals and -0) with every int8 q."""
    d_bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    d_bits = d_bits[(d_bits & 0x7C00) != 0x7C00]             # finite only
    n = d_bits.size
    q = np.tile(np.arange(-128, 128, dtype=np.int32).astype(np.int8), (n * 32 + 255) // 256)[: n * 32]
    raw = np.empty((n, 34), np.uint8)
    raw[:, 0:2] = d_bits.view(np.uint8).reshape(n, 2)
    raw[:, 2:] = q.reshape(n, 32).view(np.uint8)
    n_out = n // 8
    raw = raw[: n_out * 8].reshape(-1)
    got = host(qd.q8_0_dequantize(dev(raw), 256, n_out))
    ref = oracle.q8_0_dequantize(raw, 256, n_out)
    assert np.array_equal(f32_bits(got), f32_bits(ref))


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (5, 768), (64, 3072)])
def test_q4k_dequant_bitexact(qd, n_out, n_in):
    raw = synth.q4k_weights(21 + n_in, n_out, n_in)
    got = host(qd.q4k_dequantize(dev(raw), n_in, n_out))
    ref = oracle.q4k_dequantize(raw, n_in, n_out)
    assert np.array_equal(f32_bits(got), f32_bits(ref))


def test_q4k_dequant_bitexact_full_fp16_range(qd):
    """d and dmin over the whole finite fp16 range with random signs: the single
    rounding of the subtraction must match the oracle bit for bit."""
    rng = np.random.default_rng(77)
    n = 4096
    raw = rng.integers(0, 256, (n, 144)).astype(np.uint8)
    for off in (0, 2):
        bits = (rng.integers(0, 0x7C00, n) | (rng.integers(0, 2, n) << 15)).astype(np.uint16)
        raw[:, off:off + 2] = bits.view(np.uint8).reshape(n, 2)
    raw = raw.reshape(-1)
    got = host(qd.q4k_dequantize(dev(raw), 256 * 8, n // 8))
    ref = oracle.q4k_dequantize(raw, 256 * 8, n // 8)
    assert np.array_equal(f32_bits(got), f32_bits(ref))


def test_golden_blocks_on_gpu(qd, golden_dir):
    import json
    with open(os.path.join(golden_dir, "q8_0_blocks.json")) as f:
        cases = json.load(f)["cases"]
    raw = np.concatenate([np.frombuffer(bytes.fromhex(c["d_bytes"]) + np.asarray(c["q"], np.int8).tobytes(),
                                        np.uint8) for c in cases])
    got = host(qd.q8_0_dequantize(dev(raw), 32, len(cases)))
    exp = np.array([[float.fromhex(s) for s in c["expected"]] for c in cases], np.float32)
    assert np.array_equal(f32_bits(got), f32_bits(exp))


# ----------------------------------------------------------- Q8_0 GEMV --

GEMV_SHAPES = [(1, 32), (3, 64), (5, 96), (17, 288), (256, 512), (100, 768), (1000, 1024),
               (130, 3072), (67, 8192), (8, 2560)]


@pytest.mark.parametrize("n_out,n_in", GEMV_SHAPES)
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 7, 8])
def test_q8_0_gemv(qd, n_out, n_in, batch):
    raw = q8_weights(1000 + n_in + n_out, n_out, n_in)
    x = synth.normal_f32(2000 + batch, (batch, n_in))
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q8_0_gemv {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("n_out,n_in", [(256, 512), (3072, 8192), (77, 3072), (9, 288)])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_q8_0_gemv_residual(qd, n_out, n_in, batch):
    raw = q8_weights(3000 + n_in, n_out, n_in)
    x = synth.normal_f32(3001, (batch, n_in))
    r = synth.normal_f32(3002, (batch, n_out))
    out = host(qd.q8_0_gemv_residual(dev(raw), n_in, n_out, dev(x), dev(r)))
    ref, S = oracle.q8_0_gemv_residual(raw, n_in, n_out, x, r)
    check_f32(out, ref, S, "residual")


def test_q8_0_gemv_residual_in_place(qd):
    n_out, n_in, batch = 1000, 3072, 2
    raw = q8_weights(3100, n_out, n_in)
    x = synth.normal_f32(3101, (batch, n_in))
    r = synth.normal_f32(3102, (batch, n_out))
    rd = dev(r)
    qd.q8_0_gemv_residual(dev(raw), n_in, n_out, dev(x), rd, out=rd)
    ref, S = oracle.q8_0_gemv_residual(raw, n_in, n_out, x, r)
    check_f32(host(rd), ref, S, "residual in place")


@pytest.mark.parametrize("n_in,n_q,n_kv", [(3072, 3072, 1024), (512, 100, 20), (96, 5, 5), (288, 64, 1)])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
def test_q8_0_qkv(qd, n_in, n_q, n_kv, batch):
    wq = q8_weights(4000, n_q, n_in)
    wk = q8_weights(4001, n_kv, n_in)
    wv = q8_weights(4002, n_kv, n_in)
    x = synth.normal_f32(4003 + batch, (batch, n_in))
    q, k, v = qd.q8_0_qkv(dev(wq), dev(wk), dev(wv), n_in, n_q, n_kv, dev(x))
    (rq, rk, rv), (sq, sk, sv) = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x)
    check_f32(host(q), rq, sq, "q")
    check_f32(host(k), rk, sk, "k")
    check_f32(host(v), rv, sv, "v")


@pytest.mark.parametrize("n_out,n_in", [(8192, 3072), (100, 512), (7, 96), (33, 288)])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8])
def test_q8_0_swiglu(qd, n_out, n_in, batch):
    if n_out == 8192 and batch == 3:
        pytest.skip("covered by the smaller shapes")
    wg = q8_weights(5000 + n_in, n_out, n_in)
    wu = q8_weights(5001 + n_in, n_out, n_in)
    x = synth.normal_f32(5002 + batch, (batch, n_in))
    out = host(qd.q8_0_swiglu(dev(wg), dev(wu), n_in, n_out, dev(x)))
    r = oracle.q8_0_swiglu(wg, wu, n_in, n_out, x)
    tol = swiglu_tol(r)
    err = np.abs(out.astype(np.float64) - r["out"])
    assert np.all(err <= tol), f"worst err/tol {np.max(err / tol):.3g}"


# ----------------------------------------------------------- Q4_K GEMV --

@pytest.mark.parametrize("n_out,n_in", [(1, 256), (13, 768), (8192, 3072), (3072, 8192), (50, 2560)])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
def test_q4k_gemv(qd, n_out, n_in, batch):
    if n_out * n_in > 10_000_000 and batch not in (1, 8):
        pytest.skip("large shapes run at batch 1 and 8")
    raw = synth.q4k_weights(6000 + n_in, n_out, n_in)
    x = synth.normal_f32(6001 + batch, (batch, n_in))
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q4k {n_out}x{n_in} b{batch}")


# One batch row of Q4_K runs on the integer matrix cores for n_in = 1024 ..
# 8192 (multiples of 1024 that split into 4..16 chunks a wave): x is taken
# there as a 30-bit fixed-point number per 256 values, so inputs whose
# magnitudes differ widely within a super-block are its hard cases.
def _x_kind(kind, seed, n_in):
    x = synth.normal_f32(seed, (1, n_in))
    if kind == "outliers":      # one value 1e4 times larger in every super-block
        x[0, 17::256] *= 1e4
    elif kind == "spread":      # magnitudes over 2^-40 .. 2^40 within each block
        x *= np.exp2(np.linspace(-40, 40, n_in, dtype=np.float32)).reshape(8, -1).T.reshape(1, -1)[:, :n_in]
    elif kind == "zeros":       # whole zero super-blocks and powers of two
        x[0, :256] = 0
        x[0, 256:512] = np.exp2(np.arange(256) % 16 - 8.0) * np.where(np.arange(256) % 3, 1, -1)
    elif kind == "tiny":
        x *= np.float32(1e-30)
    elif kind == "huge":
        x *= np.float32(1e30)
    return x.astype(np.float32)


@pytest.mark.parametrize("n_in", [1024, 2048, 3072, 4096, 6144, 8192])
@pytest.mark.parametrize("kind", ["normal", "outliers", "spread", "zeros", "tiny", "huge"])
def test_q4k_one_row_matrix_core_inputs(qd, n_in, kind):
    n_out = 37   # ragged: the last 16-row group is partly padding
    raw = synth.q4k_weights(6200 + n_in, n_out, n_in)
    x = _x_kind(kind, 6201 + n_in, n_in)
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q4k one row {kind} {n_out}x{n_in}")


@pytest.mark.parametrize("n_out,n_in", [(8197, 2048), (8192, 3072), (3072, 8192), (1000, 6144), (20, 1024)])
def test_q4k_one_row_matrix_core_grids(qd, n_out, n_in):
    """Two row groups a workgroup from 512 groups on, with a spare last group
    (8197 rows: 513 groups), and the single-group grids."""
    raw = synth.q4k_weights(6220 + n_out, n_out, n_in)
    x = synth.normal_f32(6221 + n_in, (1, n_in))
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q4k one row {n_out}x{n_in}")


def test_q4k_one_row_nan_propagates(qd):
    n_out, n_in = 40, 3072
    raw = synth.q4k_weights(6210, n_out, n_in)
    x = synth.normal_f32(6211, (1, n_in))
    x[0, 700] = np.nan
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    assert np.all(np.isnan(out)), "a NaN in x must reach every output"


# One batch row with x staged in LDS: every width case of the shape table
# (whole rows per wave up to 4096 columns, K split over waves beyond; SwiGLU
# and Q4_K take it up to 4096 columns, the register shapes beyond), ragged
# row counts that leave the last workgroup partly empty, and both row counts
# per wave.
XL_SHAPES = [(13, 1024), (5, 2048), (29, 3072), (7, 4096), (9, 6144), (100, 8192), (11, 12288), (2051, 8192)]


@pytest.mark.parametrize("n_out,n_in", XL_SHAPES)
def test_one_row_lds_x_shapes(qd, n_out, n_in):
    x = synth.normal_f32(6100 + n_in, (1, n_in))
    raw8 = q8_weights(6101 + n_in, n_out, n_in)
    out = host(qd.q8_0_gemv(dev(raw8), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw8, n_in, n_out, x)
    check_f32(out, ref, S, f"q8_0 {n_out}x{n_in}")
    r = synth.normal_f32(6102 + n_in, (1, n_out))
    out = host(qd.q8_0_gemv_residual(dev(raw8), n_in, n_out, dev(x), dev(r)))
    ref, S = oracle.q8_0_gemv_residual(raw8, n_in, n_out, x, r)
    check_f32(out, ref, S, f"q8_0 residual {n_out}x{n_in}")
    raw4 = synth.q4k_weights(6103 + n_in, n_out, n_in)
    out = host(qd.q4k_gemv(dev(raw4), n_in, n_out, dev(x)))
    ref, S = oracle.q4k_gemv(raw4, n_in, n_out, x)
    check_f32(out, ref, S, f"q4k {n_out}x{n_in}")
    wu = q8_weights(6104 + n_in, n_out, n_in)
    out = host(qd.q8_0_swiglu(dev(raw8), dev(wu), n_in, n_out, dev(x)))
    r = oracle.q8_0_swiglu(raw8, wu, n_in, n_out, x)
    err = np.abs(out.astype(np.float64) - r["out"])
    assert np.all(err <= swiglu_tol(r)), f"swiglu {n_out}x{n_in}: worst err/tol {np.max(err / swiglu_tol(r)):.3g}"


@pytest.mark.parametrize("n_out,n_in", [(13, 1024), (5, 2048), (29, 3072), (7, 4096)])
def test_two_row_swiglu_lds_x_shapes(qd, n_out, n_in):
    """Two batch rows of SwiGLU up to 4096 columns: one row pair per wave, x
    staged in LDS, ragged last workgroup."""
    wg, wu = q8_weights(6120 + n_in, n_out, n_in), q8_weights(6121 + n_in, n_out, n_in)
    x = synth.normal_f32(6122 + n_in, (2, n_in))
    out = host(qd.q8_0_swiglu(dev(wg), dev(wu), n_in, n_out, dev(x)))
    r = oracle.q8_0_swiglu(wg, wu, n_in, n_out, x)
    err = np.abs(out.astype(np.float64) - r["out"])
    assert np.all(err <= swiglu_tol(r)), f"worst err/tol {np.max(err / swiglu_tol(r)):.3g}"


@pytest.mark.parametrize("n_in,n_q,n_kv", [(1024, 40, 8), (4096, 48, 16), (8192, 64, 32)])
def test_one_row_lds_x_qkv(qd, n_in, n_q, n_kv):
    wq, wk, wv = (q8_weights(6110 + i, n, n_in) for i, n in enumerate((n_q, n_kv, n_kv)))
    x = synth.normal_f32(6113, (1, n_in))
    got = [host(t) for t in qd.q8_0_qkv(dev(wq), dev(wk), dev(wv), n_in, n_q, n_kv, dev(x))]
    refs, ss = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x)
    for g, ref, S, key in zip(got, refs, ss, "qkv"):
        check_f32(g, ref, S, f"qkv {key} {n_in}")


# --------------------------------------------------------- batched GEMM --

@pytest.mark.parametrize("n_out,n_in,batch", [(16, 32, 1), (130, 96, 3), (256, 512, 128),
                                              (200, 288, 130), (128, 3072, 129), (300, 64, 512)])
def test_q8_0_gemm_batched(qd, n_out, n_in, batch):
    raw = q8_weights(7000 + n_in, n_out, n_in)
    x = synth.normal_f32(7001 + batch, (batch, n_in))
    out = host(qd.q8_0_gemm_batched(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, "gemm q8_0", rel=BF16_REL, abs_=0.0)


@pytest.mark.parametrize("n_out,n_in,batch", [(16, 32, 1), (130, 96, 3), (256, 512, 128),
                                              (200, 288, 130), (300, 64, 512)])
def test_f32_gemm_batched(qd, n_out, n_in, batch):
    w = synth.normal_f32(7100 + n_in, (n_out, n_in), 0.02)
    x = synth.normal_f32(7101 + batch, (batch, n_in))
    out = host(qd.f32_gemm_batched(dev(w), n_in, n_out, dev(x)))
    ref, S = oracle.f32_gemm(w, n_in, n_out, x)
    check_f32(out, ref, S, "gemm f32", rel=BF16_REL, abs_=0.0)


@pytest.mark.parametrize("n_out,n_in,batch", [(16, 64, 1), (130, 96, 3), (256, 512, 128), (200, 576, 130),
                                              (128, 3072, 129), (301, 64, 512), (1, 128, 2)])
def test_f32_gemm_batched_bf16_copy(qd, n_out, n_in, batch):
    """After qdec_prepare(F32) the call reads the library's bf16 copy (the
    DMA-fed kernel when n_in % 64 == 0; 96 stays on the register-staged one):
    the same bf16 products, so the same bound; after release W is read again."""
    w = synth.normal_f32(7110 + n_in, (n_out, n_in), 0.02)
    x = synth.normal_f32(7111 + batch, (batch, n_in))
    wd, xd = dev(w), dev(x)
    ref, S = oracle.f32_gemm(w, n_in, n_out, x)
    qd.prepare(wd, qd.TYPE_F32, n_in, n_out)
    try:
        out = host(qd.f32_gemm_batched(wd, n_in, n_out, xd))
        check_f32(out, ref, S, "gemm f32 bf16 copy", rel=BF16_REL, abs_=0.0)
        again = host(qd.f32_gemm_batched(wd, n_in, n_out, xd))
        assert np.array_equal(out, again), "the bf16-copy path is not reproducible"
    finally:
        qd.release(wd)
    out = host(qd.f32_gemm_batched(wd, n_in, n_out, xd))
    check_f32(out, ref, S, "gemm f32 after release", rel=BF16_REL, abs_=0.0)


# --------------------------------------------------- library behaviour --

def test_non_default_stream(qd):
    n_out, n_in = 512, 3072
    raw = q8_weights(8000, n_out, n_in)
    x = synth.normal_f32(8001, (2, n_in))
    s = torch.cuda.Stream()
    wd, xd = dev(raw), dev(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = torch.empty((2, n_out), device="cuda")
        qd.q8_0_gemv(wd, n_in, n_out, xd, out=out, stream=s)
    s.synchronize()
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out.cpu().numpy(), ref, S, "stream")


def test_cache_prepare_release_clear_and_reuse(qd):
    qd.clear_cache()
    assert qd.cache_len() == 0
    n_out, n_in = 64, 512
    a = q8_weights(8100, n_out, n_in)
    b = q8_weights(8101, n_out, n_in)
    x = synth.normal_f32(8102, (1, n_in))
    buf = dev(a)
    qd.prepare(buf, qd.TYPE_Q8_0, n_in, n_out)
    assert qd.cache_len() == 1
    qd.prepare(buf, qd.TYPE_Q8_0, n_in, n_out)      # idempotent
    assert qd.cache_len() == 1
    out = host(qd.q8_0_gemv(buf, n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(a, n_in, n_out, x)
    check_f32(out, ref, S, "prepared")
    # new bytes behind the same pointer after release: must be re-read
    qd.release(buf)
    assert qd.cache_len() == 0
    buf.copy_(dev(b))
    out = host(qd.q8_0_gemv(buf, n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(b, n_in, n_out, x)
    check_f32(out, ref, S, "after release")
    with pytest.raises(qd.QdecError):
        qd.release(dev(a))                            # never cached
    qd.clear_cache()
    assert qd.cache_len() == 0


def test_stale_pointer_needs_release(qd):
    """Documented contract: new bytes behind a cached pointer are not seen until
    qdec_release; after release the new bytes are repacked."""
    n_out, n_in = 32, 256
    a = q8_weights(8150, n_out, n_in)
    b = q8_weights(8151, n_out, n_in)
    x = synth.normal_f32(8152, (1, n_in))
    buf, xd = dev(a), dev(x)
    qd.q8_0_gemv(buf, n_in, n_out, xd)
    buf.copy_(dev(b))
    stale = host(qd.q8_0_gemv(buf, n_in, n_out, xd))
    ref_a, S_a = oracle.q8_0_gemv(a, n_in, n_out, x)
    check_f32(stale, ref_a, S_a, "cached copy still used")
    qd.release(buf)
    fresh = host(qd.q8_0_gemv(buf, n_in, n_out, xd))
    ref_b, S_b = oracle.q8_0_gemv(b, n_in, n_out, x)
    check_f32(fresh, ref_b, S_b, "after release")


def test_fail_alloc_hook(qd, monkeypatch):
    monkeypatch.setenv("QDEC_FAIL_ALLOC", "1")
    raw = dev(q8_weights(8200, 8, 64))
    with pytest.raises(qd.QdecError) as ei:
        qd.prepare(raw, qd.TYPE_Q8_0, 64, 8)
    assert ei.value.status == qd.QDEC_ENOMEM


def test_launch_counter_witness(qd):
    raw = dev(q8_weights(8300, 32, 64))
    x = dev(synth.normal_f32(8301, (1, 64)))
    before = qd.launch_count()
    qd.q8_0_gemv(raw, 64, 32, x)
    qd.q8_0_gemv(raw, 64, 32, x)
    sync()
    assert qd.launch_count() >= before + 2


# The DMA-fed Q8_0 GEMM (n_in % 64 == 0, even n_out): x rounded to bf16 in the
# stream workspace, then the kernel (2 launches), plus the slice sum when K is
# split (while the grid of 128 x 128 tiles stays at most 192 workgroups and each
# slice keeps 8 or more 64-k stages).  Ragged M and N tiles, one-stage K, odd
# tile counts and uneven slices are included; odd n_out takes the
# register-staged kernel (1 launch, no split at this size).
@pytest.mark.parametrize("n_out,n_in,batch,launches", [(2048, 256, 2048, 2), (2040, 192, 2000, 2),
                                                       (4096, 64, 1000, 2), (2048, 2048, 512, 3),
                                                       (3072, 4096, 128, 3),    # 24 tiles, 8-way split
                                                       (130, 128, 3, 2), (202, 640, 77, 2),
                                                       (66, 1024, 300, 3),      # 3 tiles, 2 slices
                                                       (1000, 1600, 9, 3),      # 8 tiles, 3 uneven slices
                                                       (129, 128, 5, 1)])       # odd n_out
def test_q8_0_gemm_pipelined(qd, n_out, n_in, batch, launches):
    raw = q8_weights(7100 + n_in, n_out, n_in)
    x = synth.normal_f32(7101 + batch, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    qd.q8_0_gemm_batched(w, n_in, n_out, xd)        # makes the stream workspace
    torch.cuda.synchronize()
    before = qd.launch_count()
    out = host(qd.q8_0_gemm_batched(w, n_in, n_out, xd))
    assert qd.launch_count() - before == launches
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, "gemm q8_0 pipelined", rel=BF16_REL, abs_=0.0)


def test_q8_0_gemm_pipelined_long_k_sampled(qd):
    """n_in = 1600: 25 stages of 64, three 8-stage unrolled blocks and a
    one-stage tail; rows sampled against the oracle."""
    n_out, n_in, batch = 4096, 1600, 1024            # 32 x 8 tiles
    raw = q8_weights(7110, n_out, n_in)
    x = synth.normal_f32(7111, (batch, n_in))
    out = host(qd.q8_0_gemm_batched(dev(raw), n_in, n_out, dev(x)))
    rng = np.random.default_rng(7112)
    row_bytes = (n_in // 32) * 34
    for b, i in zip(rng.integers(0, batch, 256), rng.integers(0, n_out, 256)):
        ref, S = oracle.q8_0_gemv(raw[i * row_bytes:(i + 1) * row_bytes], n_in, 1, x[b:b + 1])
        check_f32(out[b, i:i + 1], ref[0], S[0], f"gemm long-k b{b} i{i}", rel=BF16_REL, abs_=0.0)
    assert np.isfinite(out).all()


def test_q8_0_gemm_capture_without_workspace(qd):
    """A capture on a stream with no workspace takes the register-staged kernel
    (one launch) and still meets the bound."""
    n_out, n_in, batch = 2048, 256, 2048
    raw = q8_weights(7120, n_out, n_in)
    x = synth.normal_f32(7121, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    torch.cuda.synchronize()
    out = torch.empty((batch, n_out), device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    before = qd.launch_count()
    with torch.cuda.graph(g, stream=s):
        qd.q8_0_gemm_batched(w, n_in, n_out, xd, out=out)
    assert qd.launch_count() - before == 1
    g.replay()
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(host(out), ref, S, "gemm captured", rel=BF16_REL, abs_=0.0)
    del g


def test_graph_replay_after_workspace_growth(qd):
    """A graph captured on a stream holds the address of that stream's
    workspace.  An eager call that grows the workspace afterwards retires the
    old buffer instead of freeing it, so every replay still reads valid memory
    and matches the oracle (eager work and syncs between the replays)."""
    s = torch.cuda.Stream()
    n_out, n_in, batch = 256, 256, 128                 # DMA-fed GEMM: x in bf16 in the workspace
    raw = q8_weights(8400, n_out, n_in)
    x = synth.normal_f32(8401, (batch, n_in))
    w, xd = dev(raw), dev(x)
    out = torch.empty((batch, n_out), device=xd.device)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    with torch.cuda.stream(s):
        qd.q8_0_gemm_batched(w, n_in, n_out, xd, out=out)     # makes the small workspace
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qd.q8_0_gemm_batched(w, n_in, n_out, xd, out=out)
    # a much larger product on the same stream grows its workspace
    big_out, big_in, big_b = 4096, 4096, 512
    raw_b = q8_weights(8402, big_out, big_in)
    xb = synth.normal_f32(8403, (big_b, big_in))
    wb, xbd = dev(raw_b), dev(xb)
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    for rep in range(3):
        with torch.cuda.stream(s):
            ob = qd.q8_0_gemm_batched(wb, big_in, big_out, xbd)
            junk = torch.randn(8 << 20, device=xd.device)     # fresh allocations on the device
        s.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_f32(host(out), ref, S, f"replay {rep} after workspace growth", rel=BF16_REL, abs_=0.0)
        del junk
    rb, Sb = oracle.q8_0_gemv_f64(raw_b, big_in, big_out, xb.astype(np.float64))
    got = host(ob).astype(np.float64)
    assert np.all(np.abs(got - rb) <= BF16_REL * Sb)
    del g



def test_qdec_log_lines(tmp_path):
    """QDEC_LOG=1: a child process that prepares a weight, runs a batched GEMV
    (repacks and a workspace), releases the weight and clears the cache writes
    one '|'-keyed stderr line for each of those events."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import torch, numpy as np, quantized_decode_ggml_amd as qd, synth\n"
        "raw = synth.q8_0_weights(5, 64, 8192)[0]\n"
        "w = torch.from_numpy(raw).cuda()\n"
        "qd.prepare(w, qd.TYPE_Q8_0, 8192, 64)\n"
        "x = torch.from_numpy(synth.normal_f32(6, (6, 8192))).cuda()\n"
        "qd.q8_0_gemv(w, 8192, 64, x); torch.cuda.synchronize()\n"
        "qd.release(w); qd.clear_cache()\n")
    env = dict(os.environ, QDEC_LOG="1", PYTHONPATH=os.pathsep.join([root, os.path.join(root, "tests")]))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env, cwd=root)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("qdec|")]
    kinds = [ln.split("|")[1] for ln in lines]
    assert kinds.count("repack") == 2, lines          # row-major and tiled Q8_0 copies
    assert "type=q8_0|n_in=8192|n_out=64" in "".join(lines)
    assert "type=q8_0_tiled" in "".join(lines)
    assert kinds.count("workspace") == 1, lines       # the K slices' sums of the 6-row product
    assert kinds.count("release") == 2 and kinds[-1] == "clear_cache", lines


# 2..8 batch rows of Q4_K on the integer matrix cores (whole rows up to 4096
# columns; 6144 and 8192 in one launch up to 4 rows, as two launches of 2..4
# rows above), from the one-row kernel's tiled copy.
@pytest.mark.parametrize("n_in,batch", [(1024, 2), (1024, 8), (2048, 3), (2048, 7), (3072, 4), (3072, 8),
                                        (4096, 5), (6144, 2), (6144, 4), (6144, 5), (6144, 7), (8192, 3),
                                        (8192, 6), (8192, 8)])
def test_q4k_rows_matrix_core(qd, n_in, batch):
    n_out = 45   # ragged: the last 16-row group partly padding
    raw = synth.q4k_weights(6300 + n_in + batch, n_out, n_in)
    x = synth.normal_f32(6301 + batch, (batch, n_in))
    w = dev(raw)
    qd.prepare(w, qd.TYPE_Q4_K, n_in, n_out)
    torch.cuda.synchronize()
    before = qd.launch_count()
    out = host(qd.q4k_gemv(w, n_in, n_out, dev(x)))
    assert qd.launch_count() - before == (2 if n_in >= 6144 and batch > 4 else 1)
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q4k rows {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("kind", ["outliers", "spread", "zeros", "tiny", "huge"])
@pytest.mark.parametrize("n_out,n_in,batch", [(37, 3072, 8), (8197, 2048, 5)])
def test_q4k_rows_matrix_core_inputs(qd, kind, n_out, n_in, batch):
    raw = synth.q4k_weights(6310 + n_out, n_out, n_in)
    x = np.concatenate([_x_kind(kind, 6311 + b, n_in) for b in range(batch)])
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q4k rows {kind} {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("n_in,batch", [(3072, 6), (8192, 5)])
def test_q4k_rows_non_finite_row(qd, bad, n_in, batch):
    n_out = 40
    raw = synth.q4k_weights(6320, n_out, n_in)
    x = synth.normal_f32(6321, (batch, n_in))
    x[4, 1000] = bad
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    assert np.all(np.isnan(out[4]))
    keep = [b for b in range(batch) if b != 4]
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x[keep])
    check_f32(out[keep], ref, S, "q4k rows without a non-finite x")
