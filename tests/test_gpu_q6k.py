"""GPU parity of the Q6_K path: the dequantisation export bit for bit against
the oracle (every weight is exact in f32), and the GEMV to the f32 bound
|gpu - oracle| <= 1e-5 * S + 1e-6, S = sum_j |w_ij x_bj| from the oracle, on
the one-row matrix-core shapes (widths 1024, 2048, 3072, 4096, 6144, 8192),
the VALU paths (other widths, several batch rows, a graph captured before the
tiled copy exists), ragged row counts and the 128256 x 3072
output-projection shape.  Layout reading: the public
GGML Q6_K block (parity against real GGML files unpinned)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import check_f32, to_dev

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
    qd.clear_cache()
    yield
    qd.clear_cache()


def dev(a):
    return to_dev(a, torch)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("n_out,n_in", [(1, 256), (7, 512), (64, 3072), (300, 8192)])
def test_dequantize_bit_exact(qd, n_out, n_in):
    raw = synth.q6k_weights(9600 + n_out, n_out, n_in)
    got = host(qd.q6k_dequantize(dev(raw), n_in, n_out))
    ref = oracle.q6k_dequantize(raw, n_in, n_out)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n_out,n_in", [(8192, 3072), (3072, 8192), (77, 1024), (77, 2048), (130, 4096), (33, 6144)])
def test_gemv_one_row_fast_shapes(qd, n_out, n_in):
    raw = synth.q6k_weights(9610 + n_in, n_out, n_in)
    x = synth.normal_f32(9611, (1, n_in))
    w = dev(raw)
    qd.prepare(w, qd.TYPE_Q6_K, n_in, n_out)
    torch.cuda.synchronize()
    before = qd.launch_count()
    out = host(qd.q6k_gemv(w, n_in, n_out, dev(x)))
    assert qd.launch_count() - before == 1
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k {n_out}x{n_in}")


@pytest.mark.parametrize("n_in", [256, 768, 1024, 3072, 5120])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
def test_gemv_general_and_batches(qd, n_in, batch):
    n_out = 45
    raw = synth.q6k_weights(9620 + n_in, n_out, n_in)
    x = synth.normal_f32(9621 + batch, (batch, n_in))
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k general {n_out}x{n_in} b{batch}")


def test_gemv_extreme_quants(qd):
    """All quants 0 or 63 (q - 32 = -32 or 31) and scales at -128 / 127."""
    n_out, n_in = 20, 3072
    raw = synth.q6k_weights(9630, n_out, n_in).reshape(n_out, n_in // 256, 210)
    rng = np.random.default_rng(9631)
    raw[:, :, 0:192] = rng.choice(np.array([0, 255], np.uint8), size=raw[:, :, 0:192].shape)
    raw[:, :, 192:208] = rng.choice(np.array([0x80, 0x7F], np.uint8), size=raw[:, :, 192:208].shape)
    raw = raw.reshape(-1)
    x = synth.normal_f32(9632, (1, n_in))
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, "q6k extremes")
    got = host(qd.q6k_dequantize(dev(raw), n_in, n_out))
    assert np.array_equal(got.view(np.uint32), oracle.q6k_dequantize(raw, n_in, n_out).view(np.uint32))


def test_output_projection_shape(qd):
    """The output tensor's shape, 128256 x 3072, one row."""
    n_out, n_in = 128256, 3072
    raw = synth.q6k_weights(9640, n_out, n_in)
    x = synth.normal_f32(9641, (1, n_in))
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, "q6k 128256x3072")


# One batch row runs on the integer matrix cores for n_in = 1024, 2048, 3072,
# 4096, 6144 and 8192: x is taken there as a 30-bit fixed-point number per 16
# values (one scale group), so inputs whose magnitudes differ widely within a
# group are its hard cases.
def _x_kind(kind, seed, n_in):
    x = synth.normal_f32(seed, (1, n_in))
    if kind == "outliers":      # one value 1e4 times larger in every 16
        x[0, 5::16] *= 1e4
    elif kind == "spread":      # magnitudes over 2^-40 .. 2^40 within each group
        x *= np.exp2(np.tile(np.linspace(-40, 40, 16), n_in // 16)).astype(np.float32)
    elif kind == "zeros":       # whole zero groups and powers of two
        x[0, :256] = 0
        x[0, 256:512] = np.exp2(np.arange(256) % 16 - 8.0) * np.where(np.arange(256) % 3, 1, -1)
    elif kind == "tiny":
        x *= np.float32(1e-30)
    elif kind == "huge":
        x *= np.float32(1e30)
    return x.astype(np.float32)


@pytest.mark.parametrize("n_in", [1024, 2048, 3072, 4096, 6144, 8192])
@pytest.mark.parametrize("kind", ["normal", "outliers", "spread", "zeros", "tiny", "huge"])
def test_one_row_matrix_core_inputs(qd, n_in, kind):
    n_out = 37   # ragged: the last 16-row group is partly padding
    raw = synth.q6k_weights(9650 + n_in, n_out, n_in)
    x = _x_kind(kind, 9651 + n_in, n_in)
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k one row {kind} {n_out}x{n_in}")


@pytest.mark.parametrize("n_out,n_in", [(8197, 2048), (8192, 1024), (1000, 6144), (20, 8192), (16, 3072)])
def test_one_row_matrix_core_grids(qd, n_out, n_in):
    """Two row groups a workgroup from 512 groups on, with a spare last group
    (8197 rows: 513 groups), and single-group grids."""
    raw = synth.q6k_weights(9660 + n_out, n_out, n_in)
    x = synth.normal_f32(9661 + n_in, (1, n_in))
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k one row {n_out}x{n_in}")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_one_row_non_finite_x_propagates(qd, bad):
    n_out, n_in = 40, 3072
    raw = synth.q6k_weights(9670, n_out, n_in)
    x = synth.normal_f32(9671, (1, n_in))
    x[0, 700] = bad
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    assert np.all(np.isnan(out)), "a non-finite x must make every output NaN"


def test_one_row_deterministic(qd):
    """Fixed summation order: repeated calls give the same bits."""
    n_out, n_in = 8192, 3072
    raw = dev(synth.q6k_weights(9680, n_out, n_in))
    x = dev(synth.normal_f32(9681, (1, n_in)))
    first = host(qd.q6k_gemv(raw, n_in, n_out, x))
    for _ in range(3):
        again = host(qd.q6k_gemv(raw, n_in, n_out, x))
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_capture_before_the_tiled_copy_uses_the_valu_kernel(qd):
    """Inside a graph capture no copy can be made: with only the row-major
    copy present (a batch-2 call made it), a one-row call captured before any
    one-row call runs the VALU kernel, and the replays agree with the oracle."""
    n_out, n_in = 300, 3072
    raw = synth.q6k_weights(9690, n_out, n_in)
    w = dev(raw)
    x2 = dev(synth.normal_f32(9691, (2, n_in)))
    qd.q6k_gemv(w, n_in, n_out, x2)          # makes the row-major copy only
    torch.cuda.synchronize()
    qd.q6k_gemv(w, n_in, n_out, x2)          # finds that copy complete
    torch.cuda.synchronize()
    x = synth.normal_f32(9692, (1, n_in))
    xd = dev(x)
    out = torch.empty((1, n_out), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qd.q6k_gemv(w, n_in, n_out, xd, out=out)
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        check_f32(out.cpu().numpy(), ref, S, "q6k captured one row")
    # outside a capture the tiled copy is made, and the result agrees too
    direct = host(qd.q6k_gemv(w, n_in, n_out, xd))
    check_f32(direct, ref, S, "q6k one row after the capture")


# 2..8 batch rows take the integer matrix cores in one launch while the rows x
# width fit a workgroup's LDS (rows rounded up to 2, 4 or 8; 8 rows up to 4096
# columns, 4 up to 8192); 5..8 rows at 6144 and 8192 take two launches.
@pytest.mark.parametrize("n_in,batch", [(1024, 2), (1024, 8), (2048, 3), (2048, 7), (3072, 5), (3072, 8),
                                        (4096, 4), (6144, 2), (6144, 4), (8192, 2), (4096, 6), (8192, 3),
                                        (4096, 8), (8192, 4), (6144, 5), (6144, 8), (8192, 6), (8192, 8)])
def test_rows_matrix_core(qd, n_in, batch):
    n_out = 45   # ragged: 3 groups of 16, the last partly padding; a spare group in the last workgroup
    raw = synth.q6k_weights(9700 + n_in + batch, n_out, n_in)
    x = synth.normal_f32(9701 + batch, (batch, n_in))
    w = dev(raw)
    qd.prepare(w, qd.TYPE_Q6_K, n_in, n_out)
    torch.cuda.synchronize()
    before = qd.launch_count()
    out = host(qd.q6k_gemv(w, n_in, n_out, dev(x)))
    assert qd.launch_count() - before == (2 if n_in >= 6144 and batch > 4 else 1)
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k rows {n_out}x{n_in} b{batch}")


@pytest.mark.parametrize("kind", ["outliers", "spread", "zeros", "tiny", "huge"])
def test_rows_matrix_core_inputs(qd, kind):
    n_out, n_in, batch = 37, 3072, 8
    raw = synth.q6k_weights(9710, n_out, n_in)
    x = np.concatenate([_x_kind(kind, 9711 + b, n_in) for b in range(batch)])
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k rows {kind}")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("n_in,batch,row", [(2048, 6, 3), (8192, 7, 5)])
def test_rows_non_finite_row(qd, bad, n_in, batch, row):
    n_out = 40
    raw = synth.q6k_weights(9720, n_out, n_in)
    x = synth.normal_f32(9721, (batch, n_in))
    x[row, 500] = bad
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    assert np.all(np.isnan(out[row]))
    keep = [b for b in range(batch) if b != row]
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x[keep])
    check_f32(out[keep], ref, S, "rows without a non-finite x")


def test_rows_output_projection(qd):
    """The output tensor's shape at 4 and 8 batch rows (a batched decode step)."""
    n_out, n_in = 128256, 3072
    raw = synth.q6k_weights(9730, n_out, n_in)
    w = dev(raw)
    for batch in (4, 8):
        x = synth.normal_f32(9731 + batch, (batch, n_in))
        out = host(qd.q6k_gemv(w, n_in, n_out, dev(x)))
        ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
        check_f32(out, ref, S, f"q6k 128256x3072 b{batch}")


@pytest.mark.parametrize("n_in,batch", [(3072, 3), (3072, 5), (3072, 8), (2048, 4), (2048, 7), (1024, 8),
                                        (4096, 8)])
def test_rows_tall_ragged(qd, n_in, batch):
    """A tall matrix (2051 row groups, the last one partly padding): 4 rows take
    four row groups a workgroup and 8 rows three, so the last workgroup holds
    spare groups."""
    n_out = 2050 * 16 + 5
    raw = synth.q6k_weights(9740 + n_in + batch, n_out, n_in)
    x = synth.normal_f32(9741 + batch, (batch, n_in))
    out = host(qd.q6k_gemv(dev(raw), n_in, n_out, dev(x)))
    ref, S = oracle.q6k_gemv(raw, n_in, n_out, x)
    check_f32(out, ref, S, f"q6k {n_out}x{n_in} b{batch}")
