"""GPU parity of RMSNorm and the chained pre-norm decode block:
qdec_rmsnorm, q8_0_rmsnorm_qkv (the norm folded into the one-row product, or
normalised into scratch for several rows) and q8_0_attn_out_ffn
(h += Wo attn; h += Wd SwiGLU(RMSNorm(h))).

Every stage is checked against the oracle applied to the input the GPU stage
actually received: the normalised vector exists only in f64 on the oracle side
(oracle.rmsnorm) and its product uses S = |deq(W)| |y|; bounds as the other
f32 paths (1e-5 * S + 1e-6; SwiGLU the propagated bound).  RMSNorm alone:
|gpu - oracle| <= 1e-5 |oracle| + 1e-12 (the sum of squares and the root are
f64 on the GPU too; the scale is rounded to f32 once and applied in two f32
products)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_f32, q8_weights, swiglu_tol, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

EPS = 1e-5


@pytest.fixture(scope="module")
def qd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_decode_ggml_amd as q
    return q


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


def launches(qd, fn):
    torch.cuda.synchronize()
    before = qd.launch_count()
    r = fn()
    torch.cuda.synchronize()
    return r, qd.launch_count() - before


def norm_w(seed, n):
    return (1.0 + 0.1 * synth.normal_f32(seed, (n,))).astype(np.float32)


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 3072, 8192, 16384])
@pytest.mark.parametrize("batch", [1, 3, 8])
@pytest.mark.parametrize("inplace", [False, True])
def test_rmsnorm(qd, n, batch, inplace):
    x = synth.normal_f32(9500 + n, (batch, n)) * np.float32(3.0)
    w = norm_w(9501, n)
    xd = dev(x)
    out = xd if inplace else None
    got = host(qd.rmsnorm(xd, dev(w), EPS, out=out))
    ref = oracle.rmsnorm(x, w, EPS)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= 1e-5 * np.abs(ref) + 1e-12).all(), f"worst rel {np.max(err / (np.abs(ref) + 1e-30)):.3g}"


def test_rmsnorm_zero_row_and_large_values(qd):
    x = np.zeros((2, 512), np.float32)
    x[1] = 1e18                                 # the sum of squares (5e38) exceeds the f32 range
    w = norm_w(9510, 512)
    got = host(qd.rmsnorm(dev(x), dev(w), EPS))
    ref = oracle.rmsnorm(x, w, EPS)
    assert (got[0] == 0).all()
    assert np.allclose(got[1], ref[1], rtol=1e-5, atol=0)


@pytest.mark.parametrize("n_in", [1024, 3072, 8192])
@pytest.mark.parametrize("batch", [1, 2, 5])
def test_rmsnorm_qkv(qd, n_in, batch):
    n_q, n_kv = 384, 128
    wq, wk, wv = (q8_weights(9520 + k, n, n_in) for k, n in enumerate((n_q, n_kv, n_kv)))
    h = synth.normal_f32(9530 + batch, (batch, n_in)) * np.float32(2.0)
    w = norm_w(9531, n_in)
    dq, dk, dv = dev(wq), dev(wk), dev(wv)
    for t, rows in ((dq, n_q), (dk, n_kv), (dv, n_kv)):
        qd.prepare(t, qd.TYPE_Q8_0, n_in, rows)            # repacks are not counted below
    (q, k, v), nl = launches(qd, lambda: qd.q8_0_rmsnorm_qkv(dq, dk, dv, n_in, n_q, n_kv, dev(h), dev(w), EPS))
    if batch == 1:
        assert nl == 1                                      # folded into the one-row product
    y = oracle.rmsnorm(h, w, EPS)
    for name, got, raw, rows in (("q", q, wq, n_q), ("k", k, wk, n_kv), ("v", v, wv, n_kv)):
        ref, S = oracle.q8_0_gemv_f64(raw, n_in, rows, y)
        check_f32(host(got), ref, S, f"{name} n_in={n_in} b{batch}")


def test_rmsnorm_qkv_general_width_uses_scratch(qd):
    """n_in = 1056 is not a multiple of 1024: even one row is normalised into
    scratch first (two launches); without scratch the call is rejected."""
    n_in, n_q, n_kv = 1056, 64, 32
    wq, wk, wv = (q8_weights(9540 + k, n, n_in) for k, n in enumerate((n_q, n_kv, n_kv)))
    h = synth.normal_f32(9543, (1, n_in))
    w = norm_w(9544, n_in)
    with pytest.raises(qd.QdecError):
        qd.q8_0_rmsnorm_qkv(dev(wq), dev(wk), dev(wv), n_in, n_q, n_kv, dev(h), dev(w), EPS, scratch=0)
    scratch = torch.empty((1, n_in), device="cuda")
    dq, dk, dv = dev(wq), dev(wk), dev(wv)
    for t, rows in ((dq, n_q), (dk, n_kv), (dv, n_kv)):
        qd.prepare(t, qd.TYPE_Q8_0, n_in, rows)
    (q, k, v), nl = launches(qd, lambda: qd.q8_0_rmsnorm_qkv(dq, dk, dv, n_in, n_q, n_kv, dev(h), dev(w), EPS,
                                                             scratch=scratch))
    assert nl == 2
    y = oracle.rmsnorm(h, w, EPS)
    ref, S = oracle.q8_0_gemv_f64(wq, n_in, n_q, y)
    check_f32(host(q), ref, S, "q general width")


@pytest.mark.parametrize("batch", [1, 2, 4])
def test_attn_out_ffn_stagewise(qd, batch):
    """h1 = h + Wo attn, f = SwiGLU(RMSNorm(h1)), h2 = h1 + Wd f, each stage
    against the oracle on the GPU's own stage input (h1 from the same kernel
    run alone, f from the scratch buffer)."""
    n_embd, n_q, n_ff = 1024, 1024, 2048
    wo = q8_weights(9550, n_embd, n_q)
    wg = q8_weights(9551, n_ff, n_embd)
    wu = q8_weights(9552, n_ff, n_embd)
    wd = q8_weights(9553, n_embd, n_ff)
    g = norm_w(9554, n_embd)
    h0 = synth.normal_f32(9555 + batch, (batch, n_embd))
    attn = synth.normal_f32(9556 + batch, (batch, n_q))
    dwo, dwg, dwu, dwd, dg = dev(wo), dev(wg), dev(wu), dev(wd), dev(g)
    for t, n_in, rows in ((dwo, n_q, n_embd), (dwg, n_embd, n_ff), (dwu, n_embd, n_ff), (dwd, n_ff, n_embd)):
        qd.prepare(t, qd.TYPE_Q8_0, n_in, rows)
    h1_gpu = host(qd.q8_0_gemv_residual(dwo, n_q, n_embd, dev(attn), dev(h0)))
    hd = dev(h0)
    scratch = torch.empty((batch, n_ff + n_embd), device="cuda")
    _, nl = launches(qd, lambda: qd.q8_0_attn_out_ffn(dwo, dwg, dwu, dwd, n_embd, n_q, n_ff, hd, dev(attn), dg, EPS,
                                                     scratch=scratch))
    if batch == 1:
        assert nl == 3
    h2 = host(hd)
    f = host(scratch).reshape(-1)[:batch * n_ff].reshape(batch, n_ff)    # f is packed batch x n_ff
    # stage 1
    ref1, S1 = oracle.q8_0_gemv_residual(wo, n_q, n_embd, attn, h0)
    check_f32(h1_gpu, ref1, S1, "h1")
    # stage 2 on the GPU's h1
    y = oracle.rmsnorm(h1_gpu, g, EPS)
    r = oracle.q8_0_swiglu_f64(wg, wu, n_embd, n_ff, y)
    err = np.abs(f.astype(np.float64) - r["out"])
    assert (err <= swiglu_tol(r)).all(), f"f: worst err/tol {np.max(err / swiglu_tol(r)):.3g}"
    # stage 3 on the GPU's f and h1
    ref3, S3 = oracle.q8_0_gemv_residual(wd, n_ff, n_embd, f, h1_gpu)
    check_f32(h2, ref3, S3, "h2")


def test_layer_graph_capture_replays(qd):
    """rmsnorm_qkv + attn_out_ffn captured in one graph (4 launches at one
    row); h is reset between replays; every replay equals the eager run bit
    for bit."""
    n_embd, n_q, n_kv, n_ff = 1024, 1024, 256, 2048
    ws = {k: dev(q8_weights(9560 + i, r, c)) for i, (k, r, c) in enumerate(
        (("wq", n_q, n_embd), ("wk", n_kv, n_embd), ("wv", n_kv, n_embd), ("wo", n_embd, n_q),
         ("wg", n_ff, n_embd), ("wu", n_ff, n_embd), ("wd", n_embd, n_ff)))}
    for k, t in ws.items():
        n_in = n_q if k == "wo" else (n_ff if k == "wd" else n_embd)
        qd.prepare(t, qd.TYPE_Q8_0, n_in, t.numel() // (n_in // 32 * 34))
    g1, g2 = dev(norm_w(9570, n_embd)), dev(norm_w(9571, n_embd))
    h0 = dev(synth.normal_f32(9572, (1, n_embd)))
    h = h0.clone()
    q = torch.empty((1, n_q), device="cuda")
    k_ = torch.empty((1, n_kv), device="cuda")
    v = torch.empty((1, n_kv), device="cuda")
    scratch = torch.empty((1, n_ff + n_embd), device="cuda")

    def layer():
        qd.q8_0_rmsnorm_qkv(ws["wq"], ws["wk"], ws["wv"], n_embd, n_q, n_kv, h, g1, EPS, q_out=q, k_out=k_, v_out=v)
        qd.q8_0_attn_out_ffn(ws["wo"], ws["wg"], ws["wu"], ws["wd"], n_embd, n_q, n_ff, h, q, g2, EPS,
                             scratch=scratch)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    s.synchronize()
    eager_h, eager_q = host(h).copy(), host(q).copy()
    gr = torch.cuda.CUDAGraph()
    h.copy_(h0)
    torch.cuda.synchronize()
    before = qd.launch_count()
    with torch.cuda.graph(gr, stream=s):
        layer()
    assert qd.launch_count() - before == 4
    for r in range(3):
        h.copy_(h0)
        q.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        assert np.array_equal(host(h).view(np.uint32), eager_h.view(np.uint32)), f"replay {r} h"
        assert np.array_equal(host(q).view(np.uint32), eager_q.view(np.uint32)), f"replay {r} q"
    del gr
