"""GPU parity of the vocabulary projection with on-device top-k
(q8_0_gemv_topk): the logits match the oracle to the f32 bound; the selection
is checked bit for bit by applying the oracle's top-k to the logits the kernel
produced (the decision taken on the same f32 values); the k-th largest logits
agree with the oracle's f64 order statistics to the same bound (an order
statistic moves by at most the largest logit error).

Order (the pages fix none among ties): larger logit first, equal logits by
smaller index."""
import numpy as np
import pytest

import oracle
import synth
from helpers import F32_ABS, F32_REL, check_f32, q8_weights, to_dev

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


def check_topk(qd, raw, n_in, n_out, x, k, what):
    idx, val, logits = qd.q8_0_gemv_topk(dev(raw), n_in, n_out, dev(x), k)
    idx, val, logits = host(idx), host(val), host(logits)
    ref, S = oracle.q8_0_gemv(raw, n_in, n_out, x)
    check_f32(logits, ref, S, f"{what} logits")
    # selection on the kernel's own logits: bit-exact
    ridx, rval = oracle.topk(logits, k)
    assert np.array_equal(idx, ridx), f"{what}: indices differ from the oracle's selection"
    assert np.array_equal(val.view(np.uint32), rval.view(np.uint32)), f"{what}: values differ"
    # order statistics against the f64 logits
    tol = F32_REL * S.max(axis=1) + F32_ABS
    kth = -np.sort(-ref, axis=1)[:, :k]
    assert (np.abs(val.astype(np.float64) - kth) <= tol[:, None]).all(), f"{what}: order statistics"
    return idx


@pytest.mark.parametrize("k", [1, 8, 40, 256])
def test_vocab_projection_full_size(qd, k):
    """The 128256 x 3072 output projection (two top-k stages)."""
    n_out, n_in = 128256, 3072
    raw = q8_weights(9900, n_out, n_in)
    x = synth.normal_f32(9901, (1, n_in))
    check_topk(qd, raw, n_in, n_out, x, k, f"vocab k={k}")


@pytest.mark.parametrize("n_out", [1, 5, 4096, 4097, 8191, 12345, 70000])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_ragged_vocab_sizes(qd, n_out, batch):
    n_in = 512 if batch != 3 else 1024          # batch 3 at 1024 runs the matrix-core projection
    raw = q8_weights(9910 + n_out, n_out, n_in)
    x = synth.normal_f32(9911 + batch, (batch, n_in))
    for k in sorted({1, min(3, n_out), min(256, n_out)}):
        check_topk(qd, raw, n_in, n_out, x, k, f"n_out={n_out} b{batch} k={k}")


def test_ties_rank_by_smaller_index(qd):
    """Rows repeat a set of 50 distinct rows, so every logit occurs many times
    with identical bits; the top-k must take the smaller indices first."""
    n_out, n_in, base = 9000, 512, 50
    distinct = q8_weights(9920, base, n_in).reshape(base, -1)
    raw = np.ascontiguousarray(distinct[np.arange(n_out) % base].reshape(-1))
    x = synth.normal_f32(9921, (2, n_in))
    idx = check_topk(qd, raw, n_in, n_out, x, 256, "ties")
    _, _, logits = qd.q8_0_gemv_topk(dev(raw), n_in, n_out, dev(x), 1)
    lg = host(logits)
    assert all(np.array_equal(lg[:, i].view(np.uint32), lg[:, i % base].view(np.uint32)) for i in range(0, n_out, 97))
    for b in range(2):
        first = idx[b, 0]
        assert first < base                       # the first occurrence of the maximum


@pytest.mark.parametrize("base,k", [(3, 256), (3, 1), (1, 40)])
def test_massive_ties(qd, base, k):
    """Every logit repeats n_out/base times (one value only for base 1): the
    k-th largest key is found in the index bits, past the value's digits."""
    n_out, n_in = 12000, 256
    distinct = q8_weights(9925 + base, base, n_in).reshape(base, -1)
    raw = np.ascontiguousarray(distinct[np.arange(n_out) % base].reshape(-1))
    x = synth.normal_f32(9926, (1, n_in))
    idx = check_topk(qd, raw, n_in, n_out, x, k, f"ties base {base} k={k}")
    if base == 1:
        assert np.array_equal(idx[0], np.arange(k))


def test_staged_selection_past_the_merge_limit(qd):
    """ceil(n_out / 8192) * k above 16384: the staged multi-launch selection."""
    n_out, n_in, k = 530000, 32, 256
    raw = q8_weights(9927, n_out, n_in)
    x = synth.normal_f32(9928, (1, n_in))
    check_topk(qd, raw, n_in, n_out, x, k, "staged")


def test_graph_capture_replays(qd):
    n_out, n_in, k = 20000, 1024, 16
    raw = q8_weights(9930, n_out, n_in)
    x = synth.normal_f32(9931, (1, n_in))
    w, xd = dev(raw), dev(x)
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        e_idx, e_val, _ = qd.q8_0_gemv_topk(w, n_in, n_out, xd, k)     # makes the stream's workspace
    s.synchronize()
    e_idx, e_val = e_idx.cpu().numpy(), e_val.cpu().numpy()
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    val = torch.empty((1, k), device="cuda")
    logits = torch.empty((1, n_out), device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qd.q8_0_gemv_topk(w, n_in, n_out, xd, k, logits=logits, top_idx=idx, top_val=val)
    for r in range(3):
        idx.fill_(-1)
        val.fill_(float("nan"))
        g.replay()
        assert np.array_equal(host(idx), e_idx), f"replay {r}"
        assert np.array_equal(host(val).view(np.uint32), e_val.view(np.uint32)), f"replay {r}"
        qd.q8_0_gemv(w, n_in, n_out, xd)            # eager work between replays
    del g


def test_capture_without_workspace_is_rejected(qd):
    n_out, n_in, k = 20000, 512, 4
    w = dev(q8_weights(9940, n_out, n_in))
    x = dev(synth.normal_f32(9941, (1, n_in)))
    qd.prepare(w, qd.TYPE_Q8_0, n_in, n_out)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(qd.QdecError) as ei:
        with torch.cuda.graph(g, stream=s):
            qd.q8_0_gemv_topk(w, n_in, n_out, x, k)
    assert ei.value.status == qd.QDEC_EINVAL
    del g
    torch.cuda.synchronize()
