"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-built
blocks with values worked out by hand (tests/golden), an exhaustive comparison
with numpy's binary16 decoder, exact rational arithmetic (fractions.Fraction)
on tiny shapes, closed forms (unit vectors, zero scales, zero residual,
mathematical identities of silu), and the quantise -> dequantise error bound.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


# ------------------------------------------------------------- helpers --

def round_to_f32(v: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) binary32 value of a rational."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, -126)                       # subnormal range shares the 2^-149 grid
    ulp = Fraction(2) ** (e - 23)
    n = round(a / ulp)                     # Fraction.__round__ ties to even
    return sign * float(n * ulp)


def exact_dot(wrow, xrow):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wrow, xrow))


def block_q8_0(d_bytes_hex: str, q) -> np.ndarray:
    d = bytes.fromhex(d_bytes_hex)
    return np.frombuffer(d + np.asarray(q, np.int8).tobytes(), np.uint8).copy()


def q4k_block(d_hex, dmin_hex, scales_hex, qs) -> np.ndarray:
    raw = bytes.fromhex(d_hex) + bytes.fromhex(dmin_hex) + bytes.fromhex(scales_hex)
    raw += np.asarray(qs, np.uint8).tobytes()
    assert len(raw) == 144
    return np.frombuffer(raw, np.uint8).copy()


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "q8_0_blocks.json")) as f:
        q8 = json.load(f)
    with open(os.path.join(golden_dir, "q4k_blocks.json")) as f:
        q4 = json.load(f)
    return q8, q4


# ---------------------------------------------------------------- fp16 --

def test_fp16_exhaustive_matches_numpy():
    """All 65,536 binary16 patterns against numpy's float16 -> float32."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(f32_bits(got)[~nan], f32_bits(ref)[~nan])


def test_fp16_landmarks():
    cases = {0x0000: 0.0, 0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x7BFF: 65504.0, 0x3555: 0.333251953125}
    for h, v in cases.items():
        assert oracle.fp16_to_f32(np.array([h], np.uint16))[0] == v
    neg0 = oracle.fp16_to_f32(np.array([0x8000], np.uint16))
    assert f32_bits(neg0)[0] == 0x80000000
    assert np.isinf(oracle.fp16_to_f32(np.array([0x7C00], np.uint16))[0])


# ---------------------------------------------------------------- Q8_0 --

def test_q8_0_golden_blocks(golden):
    q8, _ = golden
    for case in q8["cases"]:
        blk = block_q8_0(case["d_bytes"], case["q"])
        got = oracle.q8_0_dequantize(blk, 32, 1)[0]
        exp = np.array([float.fromhex(s) for s in case["expected"]], np.float32)
        assert np.array_equal(f32_bits(got), f32_bits(exp)), case["name"]


def test_q8_0_row_major_block_addressing():
    """Block k of row i sits at byte (i*nb + k)*34: give every block its own d."""
    n_out, n_in = 3, 96
    nb = n_in // 32
    raw = bytearray()
    for i in range(n_out):
        for k in range(nb):
            d = np.float16(2.0 ** (i * nb + k - 4))          # distinct, exact
            raw += d.tobytes() + np.full(32, 1, np.int8).tobytes()
    w = oracle.q8_0_dequantize(np.frombuffer(bytes(raw), np.uint8), n_in, n_out)
    for i in range(n_out):
        for k in range(nb):
            assert np.all(w[i, 32 * k:32 * k + 32] == 2.0 ** (i * nb + k - 4))


def test_q8_0_zero_scale_gives_zero():
    blk = block_q8_0("0000", list(range(-16, 16)))
    w = oracle.q8_0_dequantize(blk, 32, 1)[0]
    assert np.all(w == 0.0)
    # IEEE product sign: +0 * negative q is -0, +0 * non-negative q is +0
    assert np.array_equal(np.signbit(w), np.arange(-16, 16) < 0)


def test_q8_0_dequant_exact_random():
    """Random blocks over all finite fp16 d: oracle w == d*q exactly (rational check)."""
    rng = np.random.default_rng(7)
    n = 400
    d_bits = rng.integers(0, 0x7C00, n).astype(np.uint16) | (rng.integers(0, 2, n).astype(np.uint16) << 15)
    q = rng.integers(-128, 128, (n, 32)).astype(np.int8)
    raw = np.concatenate([np.concatenate([d_bits[i:i + 1].view(np.uint8), q[i].view(np.uint8)])
                          for i in range(n)])
    w = oracle.q8_0_dequantize(raw, 32, n)
    dd = d_bits.view(np.float16).astype(np.float64)
    for i in range(0, n, 7):
        for t in range(0, 32, 5):
            assert Fraction(float(w[i, t])) == Fraction(float(dd[i])) * int(q[i, t])


# ---------------------------------------------------------------- Q4_K --

def test_q4k_scale_unpack_golden(golden):
    _, q4 = golden
    for case in q4["scale_cases"]:
        sc, m = oracle.q4k_unpack_scales(np.frombuffer(bytes.fromhex(case["scales_hex"]), np.uint8))
        assert list(sc) == case["sc"], case["name"]
        assert list(m) == case["m"], case["name"]


def _pack_scales(sc, m):
    """Encoder for the 6-bit packing (the inverse direction of the oracle's reading)."""
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return np.array(s, np.uint8)


def test_q4k_scale_pack_unpack_roundtrip():
    """Every 6-bit value in every slot survives encode -> oracle decode."""
    rng = np.random.default_rng(3)
    for trial in range(300):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        got_sc, got_m = oracle.q4k_unpack_scales(_pack_scales(sc, m))
        assert np.array_equal(got_sc, sc) and np.array_equal(got_m, m)
    # uniform random bytes <-> uniform 6-bit fields: decoding is a bijection
    seen = set()
    for b in range(256):
        s = np.zeros(12, np.uint8)
        s[8] = b
        sc, m = oracle.q4k_unpack_scales(s)
        seen.add((int(sc[4]), int(m[4])))
    assert len(seen) == 256


def test_q4k_golden_nibble_order(golden):
    _, q4 = golden
    case = next(c for c in q4["block_cases"] if c["name"] == "nibble_order")
    i = np.arange(128)
    qs = (i % 16) | ((15 - i % 16) << 4)
    w = oracle.q4k_dequantize(q4k_block(case["d_bytes"], case["dmin_bytes"], case["scales_hex"], qs), 256, 1)[0]
    e = np.arange(256)
    u = e % 64
    exp = np.where(u < 32, u % 16, 15 - u % 16).astype(np.float32)
    assert np.array_equal(w, exp)


def test_q4k_golden_scale_per_subblock(golden):
    _, q4 = golden
    case = next(c for c in q4["block_cases"] if c["name"] == "scale_per_subblock")
    w = oracle.q4k_dequantize(q4k_block(case["d_bytes"], case["dmin_bytes"], case["scales_hex"],
                                        np.full(128, 0x11, np.uint8)), 256, 1)[0]
    assert np.array_equal(w, (np.arange(256) // 32 + 1).astype(np.float32))


def test_q4k_golden_mins_only(golden):
    _, q4 = golden
    case = next(c for c in q4["block_cases"] if c["name"] == "mins_only")
    m = next(c for c in q4["scale_cases"] if c["name"] == "mixed_high_bits")["m"]
    qs = np.random.default_rng(11).integers(0, 256, 128).astype(np.uint8)
    w = oracle.q4k_dequantize(q4k_block(case["d_bytes"], case["dmin_bytes"], case["scales_hex"], qs), 256, 1)[0]
    exp = -np.array([m[e // 32] for e in range(256)], np.float32)
    assert np.array_equal(w, exp)


def test_q4k_super_block_addressing():
    """Super-block k of row i sits at byte (i*nsb + k)*144: give each its own d."""
    n_out, n_in = 2, 512
    raw = bytearray()
    sc_bytes = bytes.fromhex("010101010000000011111111")   # sc = 1 everywhere
    for idx in range(n_out * 2):
        raw += np.float16(idx + 1).tobytes() + np.float16(0).tobytes() + sc_bytes + bytes([0x11] * 128)
    w = oracle.q4k_dequantize(np.frombuffer(bytes(raw), np.uint8), n_in, n_out)
    for i in range(n_out):
        for k in range(2):
            assert np.all(w[i, 256 * k:256 * k + 256] == i * 2 + k + 1)


def test_q4k_dequant_correctly_rounded():
    """Random blocks over the whole finite fp16 range of d and dmin: the oracle's
    f32 weight equals the exact rational d*sc*q - dmin*m rounded once to f32."""
    rng = np.random.default_rng(5)
    n = 60
    raw = rng.integers(0, 256, (n, 144)).astype(np.uint8)
    for k in range(n):   # finite d, dmin with random signs and exponents
        for off in (0, 2):
            bits = np.uint16(rng.integers(0, 0x7C00)) | np.uint16(rng.integers(0, 2) << 15)
            raw[k, off:off + 2] = np.array([bits], np.uint16).view(np.uint8)
    w = oracle.q4k_dequantize(raw.reshape(-1), 256, n)
    for k in range(n):
        d = Fraction(float(raw[k, 0:2].view(np.float16)[0]))
        dmin = Fraction(float(raw[k, 2:4].view(np.float16)[0]))
        sc, m = oracle.q4k_unpack_scales(raw[k, 4:16])   # pinned separately above
        qs = raw[k, 16:]
        for e in range(0, 256, 9):
            p, u = divmod(e, 64)
            q = (qs[32 * p + u] & 15) if u < 32 else (qs[32 * p + u - 32] >> 4)
            s = 2 * p + (u >= 32)
            exact = d * int(sc[s]) * int(q) - dmin * int(m[s])
            assert float(w[k, e]) == round_to_f32(exact), (k, e)


# ------------------------------------------------------------ products --

@pytest.mark.parametrize("n_out,n_in,batch", [(1, 32, 1), (3, 64, 2), (4, 256, 3), (2, 96, 1)])
def test_q8_0_gemv_exact_rational(n_out, n_in, batch):
    raw, _ = synth.q8_0_weights(100 + n_in, n_out, n_in)
    x = synth.normal_f32(200 + n_in, (batch, n_in))
    out, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    w = oracle.q8_0_dequantize(raw, n_in, n_out)
    for b in range(batch):
        for i in range(n_out):
            ex = exact_dot(w[i], x[b])
            sa = sum(abs(Fraction(float(a)) * Fraction(float(c))) for a, c in zip(w[i], x[b]))
            assert abs(Fraction(out[b, i]) - ex) <= Fraction(1, 10 ** 15) * sa
            assert abs(Fraction(S[b, i]) - sa) <= Fraction(1, 10 ** 15) * sa


@pytest.mark.parametrize("n_out,n_in,batch", [(2, 256, 1), (3, 512, 2)])
def test_q4k_gemv_exact_rational(n_out, n_in, batch):
    raw = synth.q4k_weights(300 + n_in, n_out, n_in)
    x = synth.normal_f32(400 + n_in, (batch, n_in))
    out, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    w = oracle.q4k_dequantize(raw, n_in, n_out)
    for b in range(batch):
        for i in range(n_out):
            ex = exact_dot(w[i], x[b])
            assert abs(Fraction(out[b, i]) - ex) <= Fraction(1, 10 ** 15) * Fraction(S[b, i])


def test_gemv_unit_vectors_give_columns():
    n_out, n_in = 16, 128
    raw, _ = synth.q8_0_weights(1, n_out, n_in)
    w = oracle.q8_0_dequantize(raw, n_in, n_out)
    for j in (0, 1, 31, 32, 77, 127):
        x = np.zeros((1, n_in), np.float32)
        x[0, j] = 1.0
        out, _ = oracle.q8_0_gemv(raw, n_in, n_out, x)
        assert np.array_equal(out[0], w[:, j].astype(np.float64))
    raw4 = synth.q4k_weights(2, 4, 256)
    w4 = oracle.q4k_dequantize(raw4, 256, 4)
    for j in (0, 31, 32, 63, 64, 200, 255):
        x = np.zeros((1, 256), np.float32)
        x[0, j] = 1.0
        out, _ = oracle.q4k_gemv(raw4, 256, 4, x)
        assert np.array_equal(out[0], w4[:, j].astype(np.float64))


def test_gemv_ones_give_row_sums():
    raw, _ = synth.q8_0_weights(3, 8, 256)
    w = oracle.q8_0_dequantize(raw, 256, 8)
    out, _ = oracle.q8_0_gemv(raw, 256, 8, np.ones((1, 256), np.float32))
    for i in range(8):
        assert abs(out[0, i] - math.fsum(map(float, w[i]))) <= 1e-15 * np.sum(np.abs(w[i]))


def test_gemv_matches_numpy_f64_config0():
    """The small decode workload: Q8_0 256 x 512, batch 1, against numpy f64 matmul."""
    raw, _ = synth.q8_0_weights(synth.seed(0, 0), 256, 512)
    x = synth.normal_f32(synth.seed(0, 1), (1, 512))
    out, S = oracle.q8_0_gemv(raw, 512, 256, x)
    w = oracle.q8_0_dequantize(raw, 512, 256).astype(np.float64)
    ref = x.astype(np.float64) @ w.T
    assert np.all(np.abs(out - ref) <= 1e-13 * S)
    assert np.allclose(S, np.abs(x.astype(np.float64)[:, None, :] * w[None]).sum(-1), rtol=1e-13)


def test_quantize_dequantize_roundtrip_bound():
    """Quantise -> dequantise stays within 0.5*d_f32 + 127*|d_f32 - d_fp16| per
    element, and the dense-f32 product moves by at most sum_j bound_j |x_j|."""
    n_out, n_in = 64, 512
    raw, w = synth.q8_0_weights(9, n_out, n_in)
    deq = oracle.q8_0_dequantize(raw, n_in, n_out).astype(np.float64)
    blocks = w.reshape(n_out, -1, 32).astype(np.float64)
    d32 = (np.max(np.abs(w.reshape(n_out, -1, 32)), axis=2) / np.float32(127)).astype(np.float32)
    d16 = d32.astype(np.float16).astype(np.float64)
    bound = 0.5 * d32.astype(np.float64) + 127 * np.abs(d32.astype(np.float64) - d16)
    err = np.abs(deq.reshape(n_out, -1, 32) - blocks)
    assert np.all(err <= bound[:, :, None] * (1 + 1e-6))
    x = synth.normal_f32(10, (2, n_in))
    out, _ = oracle.q8_0_gemv(raw, n_in, n_out, x)
    dense = x.astype(np.float64) @ w.astype(np.float64).T
    per = np.repeat(bound, 32, axis=1)                 # (n_out, n_in)
    lim = np.abs(x.astype(np.float64)) @ per.T
    assert np.all(np.abs(out - dense) <= lim * (1 + 1e-6) + 1e-12)


def test_batched_equals_independent_gemvs():
    raw, _ = synth.q8_0_weights(12, 24, 128)
    x = synth.normal_f32(13, (5, 128))
    out, S = oracle.q8_0_gemv(raw, 128, 24, x)
    for b in range(5):
        o1, s1 = oracle.q8_0_gemv(raw, 128, 24, x[b:b + 1])
        assert np.array_equal(o1[0], out[b]) and np.array_equal(s1[0], S[b])


def test_f32_gemm_exact_rational_and_numpy():
    w = synth.normal_f32(14, (5, 48), 0.02)
    x = synth.normal_f32(15, (3, 48))
    out, S = oracle.f32_gemm(w, 48, 5, x)
    for b in range(3):
        for i in range(5):
            assert abs(Fraction(out[b, i]) - exact_dot(w[i], x[b])) <= Fraction(1, 10 ** 15) * Fraction(S[b, i])
    # zero padding to multiples of 16 (the pages' tensor-core path) adds zero terms only
    wp = np.zeros((16, 48), np.float32); wp[:5] = w
    xp = np.zeros((16, 48), np.float32); xp[:3] = x
    outp, _ = oracle.f32_gemm(wp, 48, 16, xp)
    assert np.array_equal(outp[:3, :5], out)


# --------------------------------------------------------------- fused --

def test_residual_closed_forms():
    raw, _ = synth.q8_0_weights(20, 32, 256)
    x = synth.normal_f32(21, (2, 256))
    r = synth.normal_f32(22, (2, 32))
    base, S = oracle.q8_0_gemv(raw, 256, 32, x)
    out0, S0 = oracle.q8_0_gemv_residual(raw, 256, 32, x, np.zeros_like(r))
    assert np.array_equal(out0, base) and np.array_equal(S0, S)
    out, _ = oracle.q8_0_gemv_residual(raw, 256, 32, x, r)
    assert np.all(np.abs(out - (base + r.astype(np.float64))) <= 1e-15 * (np.abs(out) + 1))
    zero_d = raw.reshape(32, -1, 34).copy()
    zero_d[:, :, 0:2] = 0
    outz, _ = oracle.q8_0_gemv_residual(zero_d.reshape(-1), 256, 32, x, r)
    assert np.array_equal(outz, r.astype(np.float64))


def test_qkv_is_three_gemvs_and_gqa_rows():
    n_in, n_q, n_kv = 128, 16, 4
    wq, _ = synth.q8_0_weights(30, n_q, n_in)
    wk, _ = synth.q8_0_weights(31, n_kv, n_in)
    wv, _ = synth.q8_0_weights(32, n_kv, n_in)
    x = synth.normal_f32(33, (2, n_in))
    (q, k, v), (sq, sk, sv) = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x)
    assert q.shape == (2, n_q) and k.shape == (2, n_kv) and v.shape == (2, n_kv)
    for got, s, w, n in ((q, sq, wq, n_q), (k, sk, wk, n_kv), (v, sv, wv, n_kv)):
        o, ss = oracle.q8_0_gemv(w, n_in, n, x)
        assert np.array_equal(got, o) and np.array_equal(s, ss)
    # n_kv = n_q with the same bytes for all three: three identical products
    (q2, k2, v2), _ = oracle.q8_0_qkv(wq, wq, wq, n_in, n_q, n_q, x)
    assert np.array_equal(q2, k2) and np.array_equal(k2, v2)


def _unit_weight_block_rows(n_rows, n_in, col, d_hex="003c", q=1):
    """Q8_0 rows whose only non-zero weight is q*d at column col."""
    raw = bytearray()
    for _ in range(n_rows):
        for k in range(n_in // 32):
            qq = np.zeros(32, np.int8)
            if k == col // 32:
                qq[col % 32] = q
            raw += bytes.fromhex(d_hex) + qq.tobytes()
    return np.frombuffer(bytes(raw), np.uint8).copy()


def test_silu_identities():
    """silu(0) = 0; silu(z) - silu(-z) = z; silu(ln 3) = (3/4) ln 3; silu(z) -> z
    for large z and -> 0 for very negative z."""
    assert oracle.silu(0.0) == 0.0
    for z in (0.1, 0.5, 1.0, 2.5, 7.0, 30.0):
        assert abs((oracle.silu(z) - oracle.silu(-z)) - z) <= 4e-16 * max(1.0, z)
    assert abs(oracle.silu(math.log(3.0)) - 0.75 * math.log(3.0)) <= 1e-15
    assert abs(oracle.silu(50.0) - 50.0) <= 1e-18 * 50 + 50 * math.exp(-50) * 1.01
    assert oracle.silu(-800.0) == 0.0


def test_swiglu_closed_forms():
    n_in, n_out = 64, 8
    x = np.zeros((1, n_in), np.float32)
    x[0, 5] = np.float32(math.log(3.0))
    gate = _unit_weight_block_rows(n_out, n_in, 5)               # g = x[5]
    up = _unit_weight_block_rows(n_out, n_in, 5, q=2)            # u = 2*x[5]
    r = oracle.q8_0_swiglu(gate, up, n_in, n_out, x)
    g = float(x[0, 5])
    assert np.all(r["g"] == g) and np.all(r["u"] == 2 * g)
    # silu(g)*u with g ~ ln 3: (3/4) g (2g), within the f32 rounding of ln 3
    approx = 0.75 * math.log(3.0) * 2 * math.log(3.0)
    assert np.all(np.abs(r["out"] - approx) <= 1e-6)
    # zero gate -> zero output; zero up -> zero output
    zero = _unit_weight_block_rows(n_out, n_in, 5, q=0)
    assert np.all(oracle.q8_0_swiglu(zero, up, n_in, n_out, x)["out"] == 0)
    assert np.all(oracle.q8_0_swiglu(gate, zero, n_in, n_out, x)["out"] == 0)
    # swapping gate and up changes the result (the operands are not symmetric)
    s1 = oracle.q8_0_swiglu(gate, up, n_in, n_out, x)["out"]
    s2 = oracle.q8_0_swiglu(up, gate, n_in, n_out, x)["out"]
    assert not np.allclose(s1, s2)


def test_swiglu_f64_matches_c_oracle():
    """The f64-input SwiGLU helper (used where the input is a normalised vector
    that never exists in f32) agrees with the C oracle when the input is an
    f32 vector: same g, u, S and output, to f64 rounding."""
    raw_g, _ = synth.q8_0_weights(43, 24, 320)
    raw_u, _ = synth.q8_0_weights(44, 24, 320)
    x = synth.normal_f32(45, (3, 320))
    c = oracle.q8_0_swiglu(raw_g, raw_u, 320, 24, x)
    f = oracle.q8_0_swiglu_f64(raw_g, raw_u, 320, 24, x.astype(np.float64))
    for key in ("g", "u", "Sg", "Su", "out"):
        assert np.allclose(f[key], c[key], rtol=1e-12, atol=1e-14), key


def test_swiglu_f64_closed_forms():
    """Hand-worked values with an input that is not an f32 number (ln 3 in
    f64): silu(ln 3) = (3/4) ln 3 and silu(-ln 3) = -(1/4) ln 3 exactly in real
    arithmetic, so silu(g) * u with g = y5, u = 2 y5 is (3/2) ln^2 3 and
    (1/2) ln^2 3.  The swapped product silu(u) * g is a different number
    (silu(2 ln 3) = (9/5) ln 3), so a gate/up exchange fails; so does a sign
    error inside silu (silu would become z / (1 + e^z))."""
    n_in, n_out = 64, 4
    gate = _unit_weight_block_rows(n_out, n_in, 5)               # g = y[5]
    up = _unit_weight_block_rows(n_out, n_in, 5, q=2)            # u = 2 y[5]
    ln3 = math.log(3.0)
    for y5, want in ((ln3, 1.5 * ln3 * ln3), (-ln3, 0.5 * ln3 * ln3)):
        y = np.zeros((1, n_in), np.float64)
        y[0, 5] = y5
        r = oracle.q8_0_swiglu_f64(gate, up, n_in, n_out, y)
        assert np.all(r["g"] == y5) and np.all(r["u"] == 2 * y5)
        assert np.all(np.abs(r["out"] - want) <= 1e-15 * want)
        assert np.all(r["Sg"] == abs(y5)) and np.all(r["Su"] == 2 * abs(y5))
    y = np.zeros((1, n_in), np.float64)
    y[0, 5] = ln3
    swapped = oracle.q8_0_swiglu_f64(up, gate, n_in, n_out, y)["out"]
    assert np.all(np.abs(swapped - 1.8 * ln3 * ln3) <= 1e-15 * 1.8 * ln3 * ln3)
    zero = _unit_weight_block_rows(n_out, n_in, 5, q=0)
    assert np.all(oracle.q8_0_swiglu_f64(zero, up, n_in, n_out, y)["out"] == 0)
    assert np.all(oracle.q8_0_swiglu_f64(gate, zero, n_in, n_out, y)["out"] == 0)


def test_f32_gemm_f64_matches_c_oracle_and_columns():
    """The f64 matrix-product route of the dense batched GEMM agrees with the C
    oracle's sequential f64 sums, and unit vectors pick out weight columns."""
    w = synth.normal_f32(16, (40, 96), 0.02)
    x = synth.normal_f32(17, (5, 96))
    a, sa = oracle.f32_gemm(w, 96, 40, x)
    b, sb = oracle.f32_gemm_f64(w, 96, 40, x)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    assert np.allclose(sa, sb, rtol=1e-13, atol=1e-15)
    e = np.zeros((3, 96), np.float64)
    e[0, 7] = e[1, 50] = e[2, 95] = 1.0
    cols, _ = oracle.f32_gemm_f64(w, 96, 40, e)
    for r, j in enumerate((7, 50, 95)):
        assert np.array_equal(cols[r], w[:, j].astype(np.float64))


def test_swiglu_matches_gemvs():
    raw_g, _ = synth.q8_0_weights(40, 16, 256)
    raw_u, _ = synth.q8_0_weights(41, 16, 256)
    x = synth.normal_f32(42, (3, 256))
    r = oracle.q8_0_swiglu(raw_g, raw_u, 256, 16, x)
    g, sg = oracle.q8_0_gemv(raw_g, 256, 16, x)
    u, su = oracle.q8_0_gemv(raw_u, 256, 16, x)
    assert np.array_equal(r["g"], g) and np.array_equal(r["u"], u)
    assert np.array_equal(r["Sg"], sg) and np.array_equal(r["Su"], su)
    # silu(g) = g * sigmoid(g), with sigmoid from its tanh form (a different formula)
    sig = 0.5 * (1.0 + np.tanh(0.5 * g))
    assert np.allclose(r["out"], g * sig * u, rtol=1e-13, atol=1e-300)


# ------------------------------------------------------------------ top-k --
# Reading (the pages fix no order among equal logits): larger value first,
# equal values by smaller index; -0 equals +0; NaN rejected.

def _ranks_before(a, b, v):
    """Does index a rank before index b? (stated order, written independently
    of the oracle's comparator)"""
    return v[a] > v[b] or (v[a] == v[b] and a < b)


def test_topk_hand_example():
    v = np.array([[1.0, 5.0, 3.0, 5.0, -2.0, 0.0]], np.float32)
    idx, val = oracle.topk(v, 3)
    assert idx.tolist() == [[1, 3, 2]]
    assert val.tolist() == [[5.0, 5.0, 3.0]]
    idx, _ = oracle.topk(v, 6)
    assert idx.tolist() == [[1, 3, 2, 0, 5, 4]]


def test_topk_first_maximum_is_argmax():
    rng = np.random.default_rng(71)
    v = rng.integers(-3, 4, size=(6, 50)).astype(np.float32)   # many ties
    idx, val = oracle.topk(v, 1)
    assert (idx[:, 0] == np.argmax(v, axis=1)).all()            # numpy returns the first maximum
    assert (val[:, 0] == v.max(axis=1)).all()


def test_topk_brute_force_small():
    """Every selected index ranks before every unselected one, and the list is
    in rank order; checked by pairwise comparison on tiny rows with ties."""
    rng = np.random.default_rng(72)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, n + 1))
        v = rng.choice(np.array([-1.5, 0.0, 2.0, 2.5], np.float32), size=(1, n))
        idx, val = oracle.topk(v, k)
        sel = idx[0].tolist()
        assert len(set(sel)) == k
        rest = [i for i in range(n) if i not in sel]
        assert all(_ranks_before(a, b, v[0]) for a in sel for b in rest)
        assert all(_ranks_before(sel[r], sel[r + 1], v[0]) for r in range(k - 1))
        assert (val[0] == v[0][sel]).all()


def test_topk_signed_zero_and_infinities():
    v = np.array([[-0.0, 0.0, -0.0, np.inf, -np.inf]], np.float32)
    idx, val = oracle.topk(v, 5)
    assert idx.tolist() == [[3, 0, 1, 2, 4]]
    assert np.signbit(val[0][1]) and not np.signbit(val[0][2])   # the values keep their own bits


def test_topk_batch_rows_independent():
    rng = np.random.default_rng(73)
    v = rng.standard_normal((4, 300)).astype(np.float32)
    idx, val = oracle.topk(v, 7)
    for b in range(4):
        i1, v1 = oracle.topk(v[b:b + 1], 7)
        assert (i1[0] == idx[b]).all() and (v1[0] == val[b]).all()
        assert (np.sort(v[b])[::-1][:7] == val[b]).all()


def test_topk_rejects_bad_arguments():
    v = np.zeros((1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.topk(v, 5)
    with pytest.raises(ValueError):
        oracle.topk(v, 0)
    v[0, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.topk(v, 1)


# ---------------------------------------------------------------- RMSNorm --
# Reading (the pages print no formula): out = x / sqrt(mean(x^2) + eps) * w.

def test_rmsnorm_hand_example():
    y = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32), np.array([1.0, 1.0], np.float32), 0.0)
    rms = (12.5) ** 0.5
    assert y[0, 0] == pytest.approx(3.0 / rms, rel=1e-15)
    assert y[0, 1] == pytest.approx(4.0 / rms, rel=1e-15)
    y = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32), np.array([2.0, -0.5], np.float32), 0.5)
    r = 1.0 / (12.5 + 0.5) ** 0.5
    assert y[0].tolist() == pytest.approx([3.0 * r * 2.0, 4.0 * r * -0.5], rel=1e-15)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(81)
    w = rng.standard_normal(64).astype(np.float32)
    for c in (-3.5, 0.25, 1e10):
        x = np.full((1, 64), c, np.float32)
        assert oracle.rmsnorm(x, w, 0.0)[0] == pytest.approx(np.sign(c) * w.astype(np.float64), rel=1e-14)
    assert (oracle.rmsnorm(np.zeros((2, 64), np.float32), w, 1e-5) == 0).all()


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(82)
    x = rng.standard_normal((3, 1000)).astype(np.float32)
    ones = np.ones(1000, np.float32)
    y = oracle.rmsnorm(x, ones, 0.0)
    assert np.mean(y * y, axis=1) == pytest.approx([1.0, 1.0, 1.0], rel=1e-13)
    y4 = oracle.rmsnorm(x * np.float32(4.0), ones, 0.0)
    assert np.allclose(y4, y, rtol=1e-14, atol=0)
    w = rng.standard_normal(1000).astype(np.float32)
    assert np.allclose(oracle.rmsnorm(x, w, 1e-3), oracle.rmsnorm(x, ones, 1e-3) * w, rtol=1e-14, atol=0)


def test_rmsnorm_eps_inside_the_root():
    x = np.array([[1e-3, -1e-3]], np.float32)
    y = oracle.rmsnorm(x, np.ones(2, np.float32), 1e-6)
    r = 1.0 / (float(np.float32(1e-3)) ** 2 + 1e-6) ** 0.5
    assert y[0, 0] == pytest.approx(float(np.float32(1e-3)) * r, rel=1e-14)


def test_gemv_f64_input_matches_f32_path():
    """For an input that is exactly an f32 vector, the f64-input product equals
    the C oracle's product (a different summation, so to f64 rounding)."""
    import synth
    raw, _ = synth.q8_0_weights(83, 20, 96)
    x = synth.normal_f32(84, (2, 96))
    a, sa = oracle.q8_0_gemv(raw, 96, 20, x)
    b, sb = oracle.q8_0_gemv_f64(raw, 96, 20, x.astype(np.float64))
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    assert np.allclose(sa, sb, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------- Q6_K --
# Layout reading (not on the pages): see tests/golden/q6k_blocks.json.

def _q6k_block_from_fixture(b):
    blk = np.zeros(210, np.uint8)
    for k, v in b["ql"].items():
        blk[int(k)] = v
    for k, v in b["qh"].items():
        blk[128 + int(k)] = v
    blk[192:208] = np.array(b["scales"], np.int8).view(np.uint8)
    blk[208:210] = np.frombuffer(bytes.fromhex(b["d_hex"]), np.uint8)
    return blk


def test_q6k_golden_blocks(golden_dir):
    import json
    import os
    with open(os.path.join(golden_dir, "q6k_blocks.json")) as f:
        fx = json.load(f)
    for b in fx["blocks"]:
        w = oracle.q6k_dequantize(_q6k_block_from_fixture(b), 256, 1)[0]
        for e, v in b["expect"].items():
            assert w[int(e)] == v, f"{b['name']} weight {e}: {w[int(e)]} != {v}"


def _q6k_pack(q, sc, d16):
    """Independent encoder, written per (h, l) byte rather than per weight:
    q (256,) ints 0..63, sc (16,) ints, d16 (uint16 bits) -> 210 bytes."""
    blk = np.zeros(210, np.uint8)
    for h in range(2):
        for l in range(32):
            base = 128 * h + l
            q0, q1, q2, q3 = (int(q[base + 32 * g]) for g in range(4))
            blk[64 * h + l] = (q0 & 15) | ((q2 & 15) << 4)
            blk[64 * h + 32 + l] = (q1 & 15) | ((q3 & 15) << 4)
            blk[128 + 32 * h + l] = (q0 >> 4) | ((q1 >> 4) << 2) | ((q2 >> 4) << 4) | ((q3 >> 4) << 6)
    blk[192:208] = np.asarray(sc, np.int8).view(np.uint8)
    blk[208:210] = np.array([d16], np.uint16).view(np.uint8)
    return blk


def test_q6k_encoder_round_trip():
    rng = np.random.default_rng(91)
    for _ in range(20):
        q = rng.integers(0, 64, 256)
        sc = rng.integers(-128, 128, 16)
        d = np.float16(rng.uniform(1e-3, 2.0))
        blk = _q6k_pack(q, sc, int(d.view(np.uint16)))
        w = oracle.q6k_dequantize(blk, 256, 1)[0].astype(np.float64)
        e = np.arange(256)
        group = 8 * (e // 128) + 2 * ((e % 128) // 32) + (e % 32) // 16
        ref = float(d) * sc[group] * (q - 32)
        assert np.array_equal(w, ref)          # exact: at most 23 significant bits


def test_q6k_super_block_addressing_and_zero_scale():
    rng = np.random.default_rng(92)
    rows = []
    for i in range(2):
        row = []
        for k in range(2):
            d = np.float16(0.5 * (1 + i) + 0.25 * k)
            row.append(_q6k_pack(np.full(256, 40), np.ones(16, int), int(d.view(np.uint16))))
        rows.append(np.concatenate(row))
    w = oracle.q6k_dequantize(np.concatenate(rows), 512, 2)
    for i in range(2):
        for k in range(2):
            assert (w[i, 256 * k:256 * (k + 1)] == float(np.float16(0.5 * (1 + i) + 0.25 * k)) * 8).all()
    blk = _q6k_pack(rng.integers(0, 64, 256), rng.integers(-128, 128, 16), 0)
    assert (oracle.q6k_dequantize(blk, 256, 1) == 0).all()


@pytest.mark.parametrize("n_out,n_in,batch", [(2, 256, 1), (3, 512, 2)])
def test_q6k_gemv_exact_rational(n_out, n_in, batch):
    import synth
    raw = synth.q6k_weights(93 + n_out, n_out, n_in)
    x = synth.normal_f32(94 + batch, (batch, n_in))
    out, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    W = oracle.q6k_dequantize(raw, n_in, n_out)
    for b in range(batch):
        for i in range(n_out):
            ex = exact_dot(W[i], x[b])
            assert out[b, i] == pytest.approx(float(ex), rel=1e-12, abs=1e-15)
            assert S[b, i] == pytest.approx(float(sum(abs(Fraction(float(a)) * Fraction(float(c))) for a, c in zip(W[i], x[b]))), rel=1e-12)


# ------------------------------------------------------- decode attention --
# Readings (the pages name RoPE, the KV append and GQA SDPA without formulas):
# RoPE on adjacent pairs, angle pos * base^(-2i/d); GQA head h -> kv h // group;
# softmax(scale * q.K) V.

def test_rope_hand_example_and_identity():
    x = np.array([[1.0, 0.0, 0.0, 1.0]])
    y = oracle.rope(x, 1, 10000.0)
    a1, a2 = 1.0, 10000.0 ** -0.5
    assert y[0].tolist() == pytest.approx([math.cos(a1), math.sin(a1), -math.sin(a2), math.cos(a2)], abs=1e-15)
    assert np.array_equal(oracle.rope(x, 0, 10000.0), x)


def test_rope_rotations_compose_and_keep_pair_norms():
    rng = np.random.default_rng(101)
    x = rng.standard_normal((3, 16))
    y = oracle.rope(oracle.rope(x, 7, 500000.0), 11, 500000.0)
    assert np.allclose(y, oracle.rope(x, 18, 500000.0), rtol=0, atol=1e-12)
    z = oracle.rope(x, 12345, 10000.0)
    assert np.allclose(z[:, 0::2] ** 2 + z[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2, rtol=1e-13)


def test_rope_scores_depend_on_relative_position():
    rng = np.random.default_rng(102)
    q, k = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    d1 = float(oracle.rope(q, 5, 10000.0)[0] @ oracle.rope(k, 3, 10000.0)[0])
    d2 = float(oracle.rope(q, 1002, 10000.0)[0] @ oracle.rope(k, 1000, 10000.0)[0])
    assert d1 == pytest.approx(d2, rel=1e-10)


def _caches(rng, n_kv, max_seq, d):
    return (rng.standard_normal((n_kv, max_seq, d)).astype(np.float32),
            rng.standard_normal((n_kv, max_seq, d)).astype(np.float32))


def test_attention_single_position_and_uniform_weights():
    rng = np.random.default_rng(103)
    kc, vc = _caches(rng, 2, 16, 8)
    q = rng.standard_normal((4, 8))
    out, _ = oracle.attention(q, kc, vc, 1, 0.35)
    for h in range(4):
        assert np.array_equal(out[h], vc[h // 2, 0].astype(np.float64))
    out, _ = oracle.attention(np.zeros((4, 8)), kc, vc, 10, 0.35)
    for h in range(4):
        assert np.allclose(out[h], vc[h // 2, :10].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_attention_two_positions_by_hand():
    kc = np.zeros((1, 4, 2), np.float32)
    vc = np.zeros((1, 4, 2), np.float32)
    kc[0, 1, 0] = np.float32(2.0)
    vc[0, 0] = [1.0, -2.0]
    vc[0, 1] = [3.0, 4.0]
    scale = math.log(3.0) / 2.0                # scores 0 and ln 3: weights 1/4, 3/4
    out, a = oracle.attention(np.array([[1.0, 0.0]]), kc, vc, 2, scale)
    assert out[0].tolist() == pytest.approx([0.25 * 1 + 0.75 * 3, 0.25 * -2 + 0.75 * 4], rel=1e-14)
    assert a[0].tolist() == pytest.approx([0.25 * 1 + 0.75 * 3, 0.25 * 2 + 0.75 * 4], rel=1e-14)


def test_attention_large_scores_stay_finite():
    rng = np.random.default_rng(104)
    kc, vc = _caches(rng, 1, 32, 16)
    q = 1e3 * kc[0, 17].astype(np.float64)[None, :]       # position 17 dominates by far
    out, _ = oracle.attention(q, kc, vc, 32, 1.0)
    assert np.isfinite(out).all()
    assert np.allclose(out[0], vc[0, 17], rtol=0, atol=1e-12)


def test_attention_matches_dense_softmax():
    """Against numpy's own softmax over explicitly repeated kv heads."""
    rng = np.random.default_rng(105)
    kc, vc = _caches(rng, 2, 40, 16)
    q = rng.standard_normal((6, 16))
    out, _ = oracle.attention(q, kc, vc, 33, 0.25)
    for h in range(6):
        K = kc[h // 3, :33].astype(np.float64)
        V = vc[h // 3, :33].astype(np.float64)
        s = 0.25 * (K @ q[h])
        p = np.exp(s - s.max())
        assert np.allclose(out[h], (p / p.sum()) @ V, rtol=1e-12, atol=1e-14)
