"""GPU parity of the Q6_K path: the dequantisation export bit for bit against
the oracle (every weight is exact in f32), and the GEMV to the f32 bound
|gpu - oracle| <= 1e-5 * S + 1e-6, S = sum_j |w_ij x_bj| from the oracle, on
the one-row fast shapes (widths 1024..8192 in steps of 1024 on the listed
set), the general path (other widths, several batch rows), ragged row counts
and the 128256 x 3072 output-projection shape.  Layout reading: the public
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
