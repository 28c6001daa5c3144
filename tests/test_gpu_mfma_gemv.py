"""GPU parity of the matrix-core Q8_0 GEMV paths (3..8 batch rows): which path
runs, every supported width, ragged rows and segments, activations over a wide
dynamic range (the exact three-part bf16 split of x; the per-block fixed-point
x of the integer path at widths 1024..4096), bitwise reproducibility of the K
split over workgroups and of the one-launch integer path, non-finite x, graph
capture with and without a prepared workspace, and a refused workspace
allocation.

Bar: the f32 bound, |gpu - oracle| <= 1e-5 * S + 1e-6 with S = sum_j |w x|
from the oracle (SwiGLU: the propagated bound of helpers.swiglu_tol).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_f32, q8_weights, swiglu_tol, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# widths the matrix-core path takes (n_in a multiple of 256 up to 8192): every
# K slice size (8, 16, 24, 32 blocks) and one slice per row at 256
MFMA_WIDTHS = [256, 768, 1024, 2048, 2560, 3072, 4096, 6144, 8192]


@pytest.fixture(scope="module")
def qd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_decode_ggml_amd as q
    return q


@pytest.fixture(autouse=True)
def fresh_cache(qd):
    qd.clear_cache()      # also drops the per-stream workspaces
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


@pytest.mark.parametrize("n_in,batch,expect", [(3072, 1, 1), (3072, 2, 1), (3072, 3, 1), (3072, 4, 1),
                                               (3072, 8, 1), (8192, 5, 2), (2048, 8, 1), (1024, 8, 1),
                                               (4096, 6, 1), (512, 4, 2), (2560, 8, 2), (6144, 3, 1),
                                               (8192, 4, 1), (6144, 5, 2),
                                               (256, 6, 1), (2080, 8, 1), (9216, 4, 1)])
def test_path_selection(qd, n_in, batch, expect):
    """3..8 rows at 1024, 2048, 3072 or 4096 columns, and 3..4 rows at 6144 or
    8192: the integer matrix-core kernel, whole rows in one workgroup (1
    launch).  Other supported widths
    (n_in % 256 == 0, up to 8192): the bf16 matrix-core kernel, plus the
    ordered sum of its K slices where K is split over workgroups (2 launches;
    48 rows always split K from 512 columns, 256 columns is one slice);
    otherwise the VALU kernel (1 launch)."""
    n_out = 48
    raw = q8_weights(9000 + n_in, n_out, n_in)
    x = synth.normal_f32(9001 + batch, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    out, n = launches(qd, lambda: qd.q8_0_gemv(w, n_in, n_out, xd))
    assert n == expect
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(host(out), ref, S, f"path n_in={n_in} b{batch}")


@pytest.mark.parametrize("n_in", MFMA_WIDTHS)
@pytest.mark.parametrize("n_out", [16, 77])
@pytest.mark.parametrize("batch", [3, 6, 8])
def test_gemv_widths(qd, n_in, n_out, batch):
    raw = q8_weights(9100 + n_in + n_out, n_out, n_in)
    x = synth.normal_f32(9101 + batch, (batch, n_in))
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"mfma gemv {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("batch", [3, 8])
def test_gemv_wide_dynamic_range(qd, batch):
    """Activations spread over 2^-60..2^60 (per element), so the hi, mid and lo
    parts of the split all carry weight; the bound is relative to S."""
    n_out, n_in = 40, 2048
    raw = q8_weights(9200, n_out, n_in)
    rng = np.random.default_rng(9201)
    x = (synth.normal_f32(9202, (batch, n_in)).astype(np.float64)
         * np.exp2(rng.uniform(-60, 60, size=(batch, n_in)))).astype(np.float32)
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"wide range b{batch}")


@pytest.mark.parametrize("n_q,n_kv", [(100, 20), (48, 16), (3072, 1024)])
@pytest.mark.parametrize("batch", [3, 7])
def test_qkv_ragged_segments(qd, n_q, n_kv, batch):
    """Segment boundaries inside a 16-row group of the matrix-core kernel."""
    n_in = 1024 if n_q < 3072 else 3072
    wq, wk, wv = (q8_weights(9300 + k, n, n_in) for k, n in enumerate((n_q, n_kv, n_kv)))
    x = synth.normal_f32(9310 + batch, (batch, n_in))
    (q, k, v), n = launches(qd, lambda: qd.q8_0_qkv(dev(wq), dev(wk), dev(wv), n_in, n_q, n_kv, dev(x)))
    (rq, rk, rv), (sq, sk, sv) = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x)
    check_f32(host(q), rq, sq, "q")
    check_f32(host(k), rk, sk, "k")
    check_f32(host(v), rv, sv, "v")


@pytest.mark.parametrize("n_out,n_in", [(77, 2048), (8192, 3072)])
@pytest.mark.parametrize("batch", [4, 5, 8])
def test_swiglu(qd, n_out, n_in, batch):
    g = q8_weights(9400 + n_in, n_out, n_in)
    u = q8_weights(9401 + n_in, n_out, n_in)
    x = synth.normal_f32(9402 + batch, (batch, n_in))
    out = host(qd.q8_0_swiglu(dev(g), dev(u), n_in, n_out, dev(x)))
    r = oracle.q8_0_swiglu(g, u, n_in, n_out, x)
    err = np.abs(out.astype(np.float64) - r["out"])
    assert not np.isnan(out).any()
    assert (err <= swiglu_tol(r)).all(), f"worst err/tol {np.max(err / swiglu_tol(r)):.3g}"


@pytest.mark.parametrize("batch", [3, 8])
def test_residual_in_place(qd, batch):
    n_out, n_in = 3072, 8192
    raw = q8_weights(9500, n_out, n_in)
    x = synth.normal_f32(9501, (batch, n_in))
    r = synth.normal_f32(9502, (batch, n_out))
    buf = dev(r)
    qd.q8_0_gemv_residual(dev(raw), n_in, n_out, dev(x), buf, out=buf)
    ref, S = oracle.q8_0_gemv_residual(raw, n_in, n_out, x, r)
    check_f32(host(buf), ref, S, f"residual in place b{batch}")


@pytest.mark.parametrize("n_out", [8192, 1024])
def test_graph_capture_with_workspace(qd, n_out):
    """Warm-up on the capture stream makes its workspace; the captured graph
    then uses the bf16 matrix-core path (2 launches recorded: the kernel and
    the ordered sum of its K slices) and every replay, with eager work in
    between, matches the eager result bit for bit."""
    bitwise = True
    n_in, batch = 8192, 6
    raw = q8_weights(9600, n_out, n_in)
    x = synth.normal_f32(9601, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eager = qd.q8_0_gemv(w, n_in, n_out, xd)
    s.synchronize()
    eager = eager.cpu().numpy()
    out = torch.empty((batch, n_out), device="cuda")
    g = torch.cuda.CUDAGraph()
    before = qd.launch_count()
    with torch.cuda.graph(g, stream=s):
        qd.q8_0_gemv(w, n_in, n_out, xd, out=out)
    assert qd.launch_count() - before == 2
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    for k in range(3):
        out.fill_(float("nan"))
        g.replay()
        got = host(out)
        if bitwise:
            assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {k}"
        check_f32(got, ref, S, f"replay {k}")
        qd.q8_0_gemv(w, n_in, n_out, xd)          # eager work between replays
    del g


@pytest.mark.parametrize("n_out,n_in,mode", [(3072, 8192, "residual"), (1024, 6144, "plain"), (77, 2560, "plain")])
@pytest.mark.parametrize("batch", [5, 8])
def test_k_split_bitwise_reproducible(qd, n_out, n_in, mode, batch):
    """K split over workgroups, the slices added in slice order by a second
    launch.  Five calls give the same bits, and they match the oracle to the
    f32 bound."""
    raw = q8_weights(9650 + n_out, n_out, n_in)
    x = synth.normal_f32(9651 + batch, (batch, n_in))
    r = synth.normal_f32(9652 + batch, (batch, n_out))
    w, xd, rd = dev(raw), dev(x), dev(r)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    runs = []
    for _ in range(5):
        if mode == "residual":
            out, n = launches(qd, lambda: qd.q8_0_gemv_residual(w, n_in, n_out, xd, rd))
        else:
            out, n = launches(qd, lambda: qd.q8_0_gemv(w, n_in, n_out, xd))
        assert n == 2
        runs.append(host(out))
    for k in range(1, 5):
        assert np.array_equal(runs[k].view(np.uint32), runs[0].view(np.uint32)), f"call {k} differs"
    if mode == "residual":
        ref, S = oracle.q8_0_gemv_residual(raw, n_in, n_out, x, r)
    else:
        ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(runs[0], ref, S, f"k split {mode} {n_out}x{n_in} b{batch}")


def test_graph_capture_without_workspace_falls_back(qd):
    """A capturing stream with no workspace cannot allocate one: a call that
    would split K takes the VALU kernel (1 launch recorded) and stays within
    the bound."""
    n_out, n_in, batch = 512, 8192, 8
    raw = q8_weights(9700, n_out, n_in)
    x = synth.normal_f32(9701, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    torch.cuda.synchronize()
    out = torch.empty((batch, n_out), device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    before = qd.launch_count()
    with torch.cuda.graph(g, stream=s):
        qd.q8_0_gemv(w, n_in, n_out, xd, out=out)
    assert qd.launch_count() - before == 1
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    for k in range(2):
        out.zero_()
        g.replay()
        check_f32(host(out), ref, S, f"fallback replay {k}")
    del g


@pytest.mark.parametrize("mode", ["plain", "residual", "qkv", "swiglu"])
@pytest.mark.parametrize("n_in", [512, 1024])
def test_one_slice_per_row_needs_no_workspace(qd, mode, n_in):
    """28672 rows x 512 columns fill the chip with one K slice per row of the
    bf16 kernel, and at 1024 columns the integer kernel keeps whole rows: the
    workgroups store the rows themselves (1 launch), so a capture on a stream
    that has no workspace still takes a matrix-core kernel; replays match the
    eager result bit for bit and the oracle to the f32 bound."""
    batch = 5
    n_out = 28672 if mode != "qkv" else 14336
    raws = [q8_weights(9720 + k, n_out, n_in) for k in range(3 if mode == "qkv" else 2 if mode == "swiglu" else 1)]
    x = synth.normal_f32(9725, (batch, n_in))
    r = synth.normal_f32(9726, (batch, n_out))
    ws = [dev(w) for w in raws]
    for w in ws:
        qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    xd, rd = dev(x), dev(r)

    def call(**kw):
        if mode == "plain":
            return qd.q8_0_gemv(ws[0], n_in, n_out, xd, **kw)
        if mode == "residual":
            return qd.q8_0_gemv_residual(ws[0], n_in, n_out, xd, rd, **kw)
        if mode == "swiglu":
            return qd.q8_0_swiglu(ws[0], ws[1], n_in, n_out, xd, **kw)
        return qd.q8_0_qkv(ws[0], ws[1], ws[2], n_in, n_out, n_out, xd, *kw.get("outs", ()))

    eager, n = launches(qd, call)
    assert n == 1
    eager = [host(t) for t in eager] if mode == "qkv" else [host(eager)]
    outs = [torch.empty((batch, n_out), device="cuda") for _ in eager]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    before = qd.launch_count()
    with torch.cuda.graph(g, stream=s):
        if mode == "qkv":
            call(outs=outs)
        else:
            call(out=outs[0])
    assert qd.launch_count() - before == 1
    for k in range(2):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        for o, e in zip(outs, eager):
            assert np.array_equal(host(o).view(np.uint32), e.view(np.uint32)), f"replay {k}"
    del g
    if mode == "plain":
        ref, S = oracle.q8_0_gemv(raws[0], n_in, n_out, x)
        check_f32(eager[0], ref, S, "one slice plain")
    elif mode == "residual":
        ref, S = oracle.q8_0_gemv_residual(raws[0], n_in, n_out, x, r)
        check_f32(eager[0], ref, S, "one slice residual")
    elif mode == "swiglu":
        ref = oracle.q8_0_swiglu(raws[0], raws[1], n_in, n_out, x)
        err = np.abs(eager[0].astype(np.float64) - ref["out"])
        assert (err <= swiglu_tol(ref)).all(), f"worst err/tol {np.max(err / swiglu_tol(ref)):.3g}"
    else:
        refs, ss = oracle.q8_0_qkv(raws[0], raws[1], raws[2], n_in, n_out, n_out, x)
        for e, ref, S, key in zip(eager, refs, ss, "qkv"):
            check_f32(e, ref, S, f"one slice {key}")


def test_capture_with_pending_repack_is_rejected(qd):
    """A weight used once (repack still possibly in flight) cannot be waited for
    inside a capture: the call fails cleanly instead of breaking the capture."""
    n_out, n_in = 64, 512
    w = dev(q8_weights(9750, n_out, n_in))
    x = dev(synth.normal_f32(9751, (1, n_in)))
    qd.q8_0_gemv(w, n_in, n_out, x)                  # first use: repack enqueued, not waited for
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(qd.QdecError) as ei:
        with torch.cuda.graph(g, stream=s):
            qd.q8_0_gemv(w, n_in, n_out, x)
    assert ei.value.status == qd.QDEC_EINVAL
    assert "qdec_prepare" in str(ei.value)
    del g
    torch.cuda.synchronize()


def test_workspace_allocation_refused(qd, monkeypatch):
    n_out, n_in, batch = 64, 8192, 6
    w = dev(q8_weights(9800, n_out, n_in))
    x = dev(synth.normal_f32(9801, (batch, n_in)))
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)       # the repack itself is allowed
    torch.cuda.synchronize()
    monkeypatch.setenv("QDEC_FAIL_ALLOC", "1")
    with pytest.raises(qd.QdecError) as ei:
        qd.q8_0_gemv(w, n_in, n_out, x)
    assert ei.value.status == qd.QDEC_ENOMEM


# The integer path (widths 1024 .. 4096) takes x as a 30-bit fixed-point number
# per (batch row, 32-value block), so inputs whose magnitudes differ widely
# inside a block are its hard cases.
def _x_kind(kind, seed, batch, n_in):
    x = synth.normal_f32(seed, (batch, n_in))
    if kind == "outliers":      # one value 1e4 times larger in every block
        x[:, 17::32] *= 1e4
    elif kind == "spread":      # magnitudes over 2^-40 .. 2^40 inside each block
        x *= np.exp2(np.tile(np.linspace(-40, 40, 32), n_in // 32)).astype(np.float32)
    elif kind == "zeros":       # whole zero blocks, zero rows and powers of two
        x[:, :64] = 0
        x[0, :] = 0
        x[:, 64:128] = np.exp2(np.arange(64) % 16 - 8.0) * np.where(np.arange(64) % 3, 1, -1)
    elif kind == "tiny":
        x *= np.float32(1e-30)
    elif kind == "huge":
        x *= np.float32(1e30)
    return x.astype(np.float32)


@pytest.mark.parametrize("n_in", [1024, 2048, 3072, 4096, 6144, 8192])
@pytest.mark.parametrize("kind", ["normal", "outliers", "spread", "zeros", "tiny", "huge"])
@pytest.mark.parametrize("batch", [3, 4, 5, 8])
def test_integer_path_inputs(qd, n_in, kind, batch):
    """5..8 rows at 6144 and 8192 columns run the bf16 kernel (exact split of
    x) on the same inputs; the other cases the integer kernel."""
    if kind == "tiny" and n_in >= 6144 and batch > 4:
        pytest.skip("the bf16 split is exact only above about 2^-100")
    n_out = 37   # ragged: the last 16-row group is partly padding
    raw = q8_weights(9900 + n_in, n_out, n_in)
    x = _x_kind(kind, 9901 + n_in + batch, batch, n_in)
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"integer path {kind} {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("n_out,n_in,batch", [(8197, 2048, 4), (8197, 2048, 7), (8192, 3072, 4), (8192, 3072, 7),
                                               (1000, 4096, 7), (16, 1024, 4), (5120, 3072, 7), (3072, 8192, 4),
                                               (3072, 8192, 3), (1000, 6144, 4)])
def test_integer_path_grids(qd, n_out, n_in, batch):
    """Two row groups a workgroup from 512 groups on, with a spare last group
    (8197 rows: 513 groups), and single-group grids; five calls give the same
    bits."""
    raw = q8_weights(9950 + n_out, n_out, n_in)
    x = synth.normal_f32(9951 + n_in, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    runs = []
    for _ in range(5):
        out, n = launches(qd, lambda: qd.q8_0_gemv(w, n_in, n_out, xd))
        assert n == 1
        runs.append(host(out))
    for k in range(1, 5):
        assert np.array_equal(runs[k].view(np.uint32), runs[0].view(np.uint32)), f"call {k} differs"
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(runs[0], ref, S, f"integer path {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("n_in", [1024, 3072])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_integer_path_non_finite_row(qd, n_in, bad):
    """A non-finite x makes every output of its batch row NaN; the other
    rows are unaffected."""
    n_out, batch = 40, 6
    raw = q8_weights(9960, n_out, n_in)
    x = synth.normal_f32(9961, (batch, n_in))
    x[2, 700] = bad
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    assert np.all(np.isnan(out[2])), "a non-finite x must reach every output of its row"
    keep = [b for b in range(batch) if b != 2]
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x[keep])
    check_f32(out[keep], ref, S, "rows without a non-finite x")


@pytest.mark.parametrize("n_in,batch", [(1024, 3), (1024, 8), (3072, 3), (3072, 8), (4096, 8), (8192, 4)])
def test_integer_path_residual_and_qkv(qd, n_in, batch):
    n_out = 96
    raw = q8_weights(9970 + n_in, n_out, n_in)
    x = synth.normal_f32(9971 + batch, (batch, n_in))
    r = synth.normal_f32(9972 + batch, (batch, n_out))
    out = host(qd.q8_0_gemv_residual(dev(raw), n_in, n_out, dev(x), dev(r)))
    ref, S = oracle.q8_0_gemv_residual(raw, n_in, n_out, x, r)
    check_f32(out, ref, S, f"integer residual {n_in} b{batch}")
    n_q, n_kv = 64, 16
    wq, wk, wv = (q8_weights(9980 + k, n, n_in) for k, n in enumerate((n_q, n_kv, n_kv)))
    dq, dk, dv, xd = dev(wq), dev(wk), dev(wv), dev(x)
    for t, rows in ((dq, n_q), (dk, n_kv), (dv, n_kv)):
        qd.prepare(t, qd.TYPE_Q8_0, n_in, rows)            # repacks are not counted below
    (q, k, v), n = launches(qd, lambda: qd.q8_0_qkv(dq, dk, dv, n_in, n_q, n_kv, xd))
    assert n == 1
    (rq, rk, rv), (sq, sk, sv) = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x)
    check_f32(host(q), rq, sq, "q")
    check_f32(host(k), rk, sk, "k")
    check_f32(host(v), rv, sv, "v")


@pytest.mark.parametrize("n_in", [6144, 8192])
@pytest.mark.parametrize("batch", [3, 6, 8])
def test_wide_swiglu_and_qkv(qd, n_in, batch):
    """SwiGLU at 6144 and 8192 columns takes the bf16 kernel over K slices
    (and their ordered sum) at every row count; QKV from 5 rows on."""
    n_out = 80
    g = q8_weights(9990 + n_in, n_out, n_in)
    u = q8_weights(9991 + n_in, n_out, n_in)
    x = synth.normal_f32(9992 + batch, (batch, n_in))
    dg, du, xd = dev(g), dev(u), dev(x)
    for t in (dg, du):
        qd.prepare(t, qd.TYPE_Q8_0, n_in, n_out)
    qd.q8_0_swiglu(dg, du, n_in, n_out, xd)              # makes the stream workspace
    out, n = launches(qd, lambda: qd.q8_0_swiglu(dg, du, n_in, n_out, xd))
    assert n == 2
    r = oracle.q8_0_swiglu(g, u, n_in, n_out, x)
    err = np.abs(host(out).astype(np.float64) - r["out"])
    assert (err <= swiglu_tol(r)).all(), f"worst err/tol {np.max(err / swiglu_tol(r)):.3g}"
    n_q, n_kv = 48, 16
    wq, wk, wv = (q8_weights(9995 + k, n, n_in) for k, n in enumerate((n_q, n_kv, n_kv)))
    (q, k, v) = qd.q8_0_qkv(dev(wq), dev(wk), dev(wv), n_in, n_q, n_kv, xd)
    (rq, rk, rv), (sq, sk, sv) = oracle.q8_0_qkv(wq, wk, wv, n_in, n_q, n_kv, x)
    check_f32(host(q), rq, sq, "q")
    check_f32(host(k), rk, sk, "k")
    check_f32(host(v), rv, sv, "v")


@pytest.mark.parametrize("batch,mode", [(3, "plain"), (4, "residual"), (5, "plain"), (8, "plain"),
                                        (6, "residual"), (8, "residual")])
def test_integer_path_tall(qd, batch, mode):
    """A tall product at 3072 columns (2051 row groups): 5..8 rows take four
    row groups a workgroup of 4 waves x 24 blocks (three spare groups in the
    last workgroup), 3..4 rows two row groups of 6 waves; one launch, no
    workspace."""
    n_in, n_out = 3072, 2050 * 16 + 5
    raw = q8_weights(9990 + batch, n_out, n_in)
    x = synth.normal_f32(9991 + batch, (batch, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    if mode == "plain":
        out, n = launches(qd, lambda: qd.q8_0_gemv(w, n_in, n_out, xd))
        ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    else:
        r = synth.normal_f32(9992 + batch, (batch, n_out))
        out, n = launches(qd, lambda: qd.q8_0_gemv_residual(w, n_in, n_out, xd, dev(r)))
        ref, S = oracle.q8_0_gemv_residual(raw, n_in, n_out, x, r)
    assert n == 1
    check_f32(host(out), ref, S, f"integer tall {mode} {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_integer_path_tall_non_finite_row(qd, bad):
    n_in, n_out, batch = 3072, 2048 * 16, 7
    raw = q8_weights(9995, n_out, n_in)
    x = synth.normal_f32(9996, (batch, n_in))
    x[5, 3000] = bad
    out = host(qd.q8_0_gemv(dev(raw), n_in, n_out, dev(x)))
    assert np.all(np.isnan(out[5]))
    keep = [b for b in range(batch) if b != 5]
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x[keep])
    check_f32(out[keep], ref, S, "tall rows without a non-finite x")
