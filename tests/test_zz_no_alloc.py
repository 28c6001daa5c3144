"""The allocation-free entry point q8_0_gemv_topk_noalloc, called through the
C ABI, against q8_0_gemv_topk: same logits bit for bit and the same top-k, on
two calls in a row (the second smaller), plus its refusals."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from helpers import to_dev

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


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(qd, w, n_in, n_out, x, k, logits, idx, val, stream):
    return qd.lib.q8_0_gemv_topk_noalloc(_ptr(w), n_in, n_out, x.shape[0], _ptr(x), k, _ptr(logits), _ptr(idx),
                                         _ptr(val), ctypes.c_void_p(stream.cuda_stream))


# (n_out, n_in, batch, k, seed); 3..8 rows take a matrix-core projection: at
# 1024..4096 columns whole rows stay in one workgroup, at 2560 columns (and
# 6144, 8192 from 5 rows) the K slices' sums live in the scratch (added in a
# fixed order, so the logits are reproducible bit for bit); more than 4096
# logits use the candidate lists in the scratch
@pytest.mark.parametrize("cases", [[(50000, 3072, 4, 40, 91), (3000, 1024, 2, 7, 92)],
                                   [(40000, 3072, 8, 256, 93), (9000, 2048, 3, 1, 94)],
                                   [(6000, 2560, 6, 40, 95), (5000, 2560, 3, 3, 96)]])
def test_noalloc_matches_allocating_entry_point(qd, cases):
    stream = torch.cuda.current_stream()
    for n_out, n_in, batch, k, seed in cases:
        raw = synth.q8_0_weights(seed, n_out, n_in)[0]
        x = synth.normal_f32(seed + 1, (batch, n_in))
        w, xd = to_dev(raw, torch), to_dev(x, torch)
        qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
        ref_idx, ref_val, ref_logits = qd.q8_0_gemv_topk(w, n_in, n_out, xd, k)
        logits = torch.full((batch, n_out), float("nan"), device=xd.device)
        idx = torch.full((batch, k), -1, dtype=torch.int32, device=xd.device)
        val = torch.full((batch, k), float("nan"), device=xd.device)
        before = qd.launch_count()
        rc = _noalloc(qd, w, n_in, n_out, xd, k, logits, idx, val, stream)
        assert rc == 0, qd.last_error()
        assert qd.launch_count() > before
        torch.cuda.synchronize()
        got_l, want_l = logits.cpu().numpy(), ref_logits.cpu().numpy()
        assert np.array_equal(got_l.view(np.uint32), want_l.view(np.uint32)), f"logits differ at {n_out}x{n_in} b{batch}"
        assert np.array_equal(idx.cpu().numpy(), ref_idx.cpu().numpy())
        assert np.array_equal(val.cpu().numpy().view(np.uint32), ref_val.cpu().numpy().view(np.uint32))
        # and the selection itself against the oracle's top-k of these logits
        o_idx, o_val = oracle.topk(got_l, k)
        assert np.array_equal(idx.cpu().numpy(), o_idx)
        qd.release(w)


def test_noalloc_refusals(qd):
    stream = torch.cuda.current_stream()
    n_out, n_in = 512, 256
    raw = synth.q8_0_weights(95, n_out, n_in)[0]
    w = to_dev(raw, torch)
    x = to_dev(synth.normal_f32(96, (1, n_in)), torch)
    logits = torch.empty((1, n_out), device=x.device)
    idx = torch.empty((1, 4), dtype=torch.int32, device=x.device)
    val = torch.empty((1, 4), device=x.device)
    before = qd.launch_count()
    # no repacked copy: refused, nothing made
    assert _noalloc(qd, w, n_in, n_out, x, 4, logits, idx, val, stream) == qd.QDEC_EINVAL
    assert "qdec_prepare" in qd.last_error()
    assert qd.cache_len() == 0
    # more scratch than the static array holds: refused before anything runs
    big_out = 4_000_000
    xb = to_dev(synth.normal_f32(97, (8, n_in)), torch)
    rc = qd.lib.q8_0_gemv_topk_noalloc(_ptr(w), n_in, big_out, 8, _ptr(xb), 256, _ptr(logits), _ptr(idx), _ptr(val),
                                       ctypes.c_void_p(stream.cuda_stream))
    assert rc == qd.QDEC_EINVAL and "static array" in qd.last_error()
    assert qd.launch_count() == before
