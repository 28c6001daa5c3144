"""GPU parity of the decode attention path (row f4): RoPE + KV append, and
GQA softmax attention over the f32 cache, each against the oracle on the
GPU's own inputs.

Bounds: RoPE output |gpu - oracle| <= 2^-23 |x|_pair + 1e-30 (f64 angle and
trig, one rounding to f32).  Attention: scores are f32 dot products of d
terms, so each score may be off by e_s = scale * (d + 1) * 2^-24 *
max_t sum_j |q_j K_tj|; a weight then moves by at most 2 e_s relative and
the output by (2 e_s + 1e-5) * A + 1e-7, A = sum_t p_t |V_t| (the f32 sums
over <= 256 positions per chunk and <= 64 chunks stay far below 1e-5)."""
import numpy as np
import pytest

import oracle
from helpers import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_decode_ggml_amd as q
    return q


def dev(a):
    return to_dev(a, torch)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def attention_tol(q, kc, n_ctx, scale, group, a_abs):
    d = q.shape[1]
    worst = 0.0
    for h in range(q.shape[0]):
        K = np.abs(kc[h // group, :n_ctx].astype(np.float64))
        worst = max(worst, float((K @ np.abs(q[h].astype(np.float64))).max()))
    e_s = scale * (d + 1) * 2.0 ** -24 * worst
    return (2 * e_s + 1e-5) * a_abs + 1e-7


@pytest.mark.parametrize("pos", [0, 1, 37, 4095, 8191])
@pytest.mark.parametrize("d,n_head,n_kv,base", [(128, 24, 8, 500000.0), (64, 8, 8, 10000.0)])
def test_rope_append(qd, pos, d, n_head, n_kv, base):
    rng = np.random.default_rng(9700 + pos + d)
    max_seq = 8192
    q = rng.standard_normal((n_head, d)).astype(np.float32)
    k = rng.standard_normal((n_kv, d)).astype(np.float32)
    v = rng.standard_normal((n_kv, d)).astype(np.float32)
    kc = torch.zeros((n_kv, max_seq, d), device="cuda")
    vc = torch.zeros((n_kv, max_seq, d), device="cuda")
    qd_, kd = dev(q), dev(k)
    qd.rope_kv_append(qd_, kd, dev(v), pos, base, kc, vc)
    for got, src in ((host(qd_), q), (host(kd), k)):
        ref = oracle.rope(src, pos, base)
        pair = np.repeat(np.hypot(src[:, 0::2].astype(np.float64), src[:, 1::2].astype(np.float64)), 2, axis=1)
        assert (np.abs(got - ref) <= 2.0 ** -23 * pair + 1e-30).all()
    kch, vch = host(kc), host(vc)
    assert np.array_equal(kch[:, pos], host(kd))
    assert np.array_equal(vch[:, pos], v)
    mask = np.ones(max_seq, bool)
    mask[pos] = False
    assert (kch[:, mask] == 0).all() and (vch[:, mask] == 0).all()


@pytest.mark.parametrize("n_ctx", [1, 2, 63, 256, 257, 1000, 4096, 8192])
@pytest.mark.parametrize("d,n_head,n_kv", [(128, 24, 8), (64, 16, 1), (128, 8, 8)])
def test_attention(qd, n_ctx, d, n_head, n_kv):
    rng = np.random.default_rng(9800 + n_ctx + d + n_head)
    max_seq = 8192
    kc = rng.standard_normal((n_kv, max_seq, d)).astype(np.float32)
    vc = rng.standard_normal((n_kv, max_seq, d)).astype(np.float32)
    q = (2.0 * rng.standard_normal((n_head, d))).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    got = host(qd.attention_decode(dev(q), dev(kc), dev(vc), n_ctx, scale))
    ref, a_abs = oracle.attention(q, kc, vc, n_ctx, scale)
    tol = attention_tol(q, kc, n_ctx, scale, n_head // n_kv, a_abs)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= tol).all(), f"worst err/tol {np.max(err / tol):.3g}"


@pytest.mark.parametrize("n_ctx,d,n_head,n_kv", [(3000, 128, 32, 4), (2049, 64, 12, 2), (130, 64, 12, 2)])
def test_attention_group_sizes(qd, n_ctx, d, n_head, n_kv):
    """The specialised kernels for 8 and 6 query heads a kv head, on ragged
    contexts either side of the 64/128-position chunk switch, with the cache
    longer than the context."""
    rng = np.random.default_rng(9900 + n_ctx + d + n_head)
    max_seq = n_ctx + 77
    kc = rng.standard_normal((n_kv, max_seq, d)).astype(np.float32)
    vc = rng.standard_normal((n_kv, max_seq, d)).astype(np.float32)
    q = (2.0 * rng.standard_normal((n_head, d))).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    got = host(qd.attention_decode(dev(q), dev(kc), dev(vc), n_ctx, scale))
    ref, a_abs = oracle.attention(q, kc, vc, n_ctx, scale)
    tol = attention_tol(q, kc, n_ctx, scale, n_head // n_kv, a_abs)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= tol).all(), f"worst err/tol {np.max(err / tol):.3g}"


def test_attention_peaked_and_flat(qd):
    """One position far above the rest (weights ~ one-hot), and q = 0 (flat
    weights: the mean of V over n_ctx)."""
    d, n_head, n_kv, max_seq, n_ctx = 128, 8, 2, 2048, 1500
    rng = np.random.default_rng(9900)
    kc = rng.standard_normal((n_kv, max_seq, d)).astype(np.float32)
    vc = rng.standard_normal((n_kv, max_seq, d)).astype(np.float32)
    q = np.zeros((n_head, d), np.float32)
    got = host(qd.attention_decode(dev(q), dev(kc), dev(vc), n_ctx, 0.1))
    for h in range(n_head):
        assert np.allclose(got[h], vc[h // 4, :n_ctx].astype(np.float64).mean(axis=0), rtol=0, atol=2e-6)
    q = (30.0 * kc[np.arange(n_head) // 4, 777]).astype(np.float32)
    got = host(qd.attention_decode(dev(q), dev(kc), dev(vc), n_ctx, 1.0))
    ref, a_abs = oracle.attention(q, kc, vc, n_ctx, 1.0)
    tol = attention_tol(q, kc, n_ctx, 1.0, 4, a_abs)
    assert (np.abs(got - ref) <= tol).all()


def test_block_step_with_attention(qd):
    """rope_kv_append then attention over positions 0..pos, as a decode step
    runs them; the attention input is the GPU's rotated q and its caches."""
    d, n_head, n_kv, max_seq, pos = 128, 24, 8, 4096, 2999
    rng = np.random.default_rng(9910)
    kc = dev(rng.standard_normal((n_kv, max_seq, d)).astype(np.float32))
    vc = dev(rng.standard_normal((n_kv, max_seq, d)).astype(np.float32))
    q = dev(rng.standard_normal((n_head, d)).astype(np.float32))
    k = dev(rng.standard_normal((n_kv, d)).astype(np.float32))
    v = dev(rng.standard_normal((n_kv, d)).astype(np.float32))
    qd.rope_kv_append(q, k, v, pos, 500000.0, kc, vc)
    scale = 1.0 / np.sqrt(d)
    got = host(qd.attention_decode(q, kc, vc, pos + 1, scale))
    qh, kch, vch = host(q), host(kc), host(vc)
    ref, a_abs = oracle.attention(qh, kch, vch, pos + 1, scale)
    tol = attention_tol(qh, kch, pos + 1, scale, 3, a_abs)
    assert (np.abs(got - ref) <= tol).all()
