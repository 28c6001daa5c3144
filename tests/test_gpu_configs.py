"""The five workload configurations at full size, in the launch configurations
bench.py times, against the oracle, every output (the batched GEMMs through the oracle's exact
dequantisation and an f64 matrix product).

Inputs follow the recipes of the workload definitions: Q8_0 weights from
W ~ N(0, 0.02) quantised per 32-block, Q4_K with uniform random codes and
d, dmin uniform on [1e-4, 1e-3], activations and residuals N(0, 1); seed
1000*config + index."""
import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_REL, F32_ABS, F32_REL, check_f32, swiglu_tol, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_decode_ggml_amd as q
    q.clear_cache()
    yield q
    q.clear_cache()


@pytest.fixture(autouse=True)
def fresh_cache(qd):
    qd.clear_cache()
    yield
    qd.clear_cache()


def dev(a):
    return to_dev(a, torch)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def q8(cfg, idx, n_out, n_in):
    return synth.q8_0_weights(synth.seed(cfg, idx), n_out, n_in)[0]


def test_config0_small_gemv(qd):
    raw = q8(0, 0, 256, 512)
    x = synth.normal_f32(synth.seed(0, 1), (1, 512))
    out = host(qd.q8_0_gemv(dev(raw), 512, 256, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, 512, 256, x)
    check_f32(out, ref, S, "config 0")


def test_config1_decode_layer(qd):
    n_in, n_q, n_kv, n_ff = 3072, 3072, 1024, 8192
    wq, wk, wv = q8(1, 0, n_q, n_in), q8(1, 1, n_kv, n_in), q8(1, 2, n_kv, n_in)
    up, down = q8(1, 3, n_ff, n_in), q8(1, 4, n_in, n_ff)
    xq = synth.normal_f32(synth.seed(1, 5), (1, n_in))
    xu = synth.normal_f32(synth.seed(1, 6), (1, n_in))
    xd = synth.normal_f32(synth.seed(1, 7), (1, n_ff))
    r = synth.normal_f32(synth.seed(1, 8), (1, n_in))
    q, k, v = qd.q8_0_qkv(dev(wq), dev(wk), dev(wv), n_in, n_q, n_kv, dev(xq))
    (rq, rk, rv), (sq, sk, sv) = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, xq)
    for got, ref, S, nm in ((q, rq, sq, "q"), (k, rk, sk, "k"), (v, rv, sv, "v")):
        check_f32(host(got), ref, S, f"config 1 {nm}")
    out = host(qd.q8_0_gemv(dev(up), n_in, n_ff, dev(xu)))
    ref, S = oracle.q8_0_gemv(up, n_in, n_ff, xu)
    check_f32(out, ref, S, "config 1 up")
    out = host(qd.q8_0_gemv_residual(dev(down), n_ff, n_in, dev(xd), dev(r)))
    ref, S = oracle.q8_0_gemv_residual(down, n_ff, n_in, xd, r)
    check_f32(out, ref, S, "config 1 down+residual")


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_config2_swiglu_chain(qd, batch):
    """x -> fused SwiGLU -> mid (stays on the device) -> down + residual."""
    n_in, n_ff = 3072, 8192
    wg, wu, wd = q8(2, 0, n_ff, n_in), q8(2, 1, n_ff, n_in), q8(2, 2, n_in, n_ff)
    x = synth.normal_f32(synth.seed(2, 3) + 10 * batch, (batch, n_in))
    r = synth.normal_f32(synth.seed(2, 4) + 10 * batch, (batch, n_in))
    mid = qd.q8_0_swiglu(dev(wg), dev(wu), n_in, n_ff, dev(x))
    out = qd.q8_0_gemv_residual(dev(wd), n_ff, n_in, mid, dev(r))
    mid_h, out_h = host(mid), host(out)
    # stage 1: the SwiGLU expansion
    ro = oracle.q8_0_swiglu(wg, wu, n_in, n_ff, x)
    tol_mid = swiglu_tol(ro)
    assert np.all(np.abs(mid_h - ro["out"]) <= tol_mid)
    # stage 2: the down projection of the GPU's own mid
    ref2, S2 = oracle.q8_0_gemv_residual(wd, n_ff, n_in, mid_h, r)
    check_f32(out_h, ref2, S2, "config 2 down(mid_gpu)")
    # end to end: the oracle's own chain, with the first stage's bound carried
    ref_e, S_e = oracle.q8_0_gemv_residual(wd, n_ff, n_in, ro["out"].astype(np.float32), r)
    absw = np.abs(oracle.q8_0_dequantize(wd, n_ff, n_in).astype(np.float64))
    carry = tol_mid @ absw.T                                    # (batch, n_in)
    # f32 rounding of the oracle's mid, carried the same way
    carry += (np.abs(ro["out"]) * 2.0 ** -24) @ absw.T
    err = np.abs(out_h - ref_e)
    assert np.all(err <= F32_REL * S_e + carry + F32_ABS)


def check_every_output(got, ref, S, what):
    """All batch x n_out outputs against the bf16-MFMA bound 5e-3 * S."""
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape and np.isfinite(got).all(), what
    err = np.abs(got - ref)
    bad = err > BF16_REL * S
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside 5e-3*S; worst err/S="
                           f"{np.max(err / S):.3g} at {np.unravel_index(np.argmax(err / S), err.shape)}")


@pytest.mark.parametrize("batch", [128, 512])
@pytest.mark.parametrize("which", ["up", "down"])
def test_config3_batched_gemm_q8_0(qd, batch, which):
    """Every output of the full-size product against the oracle's exact
    dequantisation followed by an f64 matrix product."""
    n_out, n_in = (8192, 3072) if which == "up" else (3072, 8192)
    raw = q8(3, 0 if which == "up" else 1, n_out, n_in)
    x = synth.normal_f32(synth.seed(3, 2) + batch, (batch, n_in))
    out = host(qd.q8_0_gemm_batched(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv_f64(raw, n_in, n_out, x.astype(np.float64))
    check_every_output(out, ref, S, f"q8_0 gemm {which} B{batch}")


@pytest.mark.parametrize("bf16_copy", [False, True])
@pytest.mark.parametrize("batch", [128, 512])
@pytest.mark.parametrize("which", ["up", "down"])
def test_config3_batched_gemm_dense_f32(qd, batch, which, bf16_copy):
    """W read in place, and W's bf16 copy (qdec_prepare) on the DMA-fed kernel."""
    n_out, n_in = (8192, 3072) if which == "up" else (3072, 8192)
    w = synth.normal_f32(synth.seed(3, 10 + (which == "down")), (n_out, n_in), 0.02)
    x = synth.normal_f32(synth.seed(3, 12) + batch, (batch, n_in))
    wd = dev(w)
    if bf16_copy:
        qd.prepare(wd, qd.TYPE_F32, n_in, n_out)
    try:
        out = host(qd.f32_gemm_batched(wd, n_in, n_out, dev(x)))
    finally:
        if bf16_copy:
            qd.release(wd)
    ref, S = oracle.f32_gemm_f64(w, n_in, n_out, x)
    check_every_output(out, ref, S, f"f32 gemm {which} B{batch}{' bf16 copy' if bf16_copy else ''}")


@pytest.mark.parametrize("shape", [(8192, 3072), (3072, 8192)])
def test_config4_q4k_gemv(qd, shape):
    n_out, n_in = shape
    raw = synth.q4k_weights(synth.seed(4, 0 if n_out == 8192 else 1), n_out, n_in)
    x = synth.normal_f32(synth.seed(4, 2), (1, n_in))
    out = host(qd.q4k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q4k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"config 4 q4k {shape}")


def test_config4_vocab_projection(qd):
    n_out, n_in = 128256, 3072
    raw = q8(4, 3, n_out, n_in)
    x = synth.normal_f32(synth.seed(4, 4), (1, n_in))
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, "config 4 vocab")
