"""C-ABI checks that need no GPU: the library loads, exports every function
include/qdec.h declares, and rejects invalid arguments with QDEC_EINVAL before
it makes any HIP call."""
import ctypes

import pytest

qd = pytest.importorskip("quantized_decode_ggml_amd")

FAKE = 0x10000       # never dereferenced: every call below fails validation first


def test_every_declared_function_is_exported():
    names = qd.declared_functions()
    assert len(names) >= 17
    for name in names:
        assert hasattr(qd.lib, name), f"{name} declared in qdec.h but not exported"
    for core in ("q8_0_gemv", "q8_0_qkv", "q8_0_swiglu", "q8_0_gemv_residual", "q4k_gemv",
                 "q8_0_gemm_batched"):
        assert core in names


def test_initial_state():
    assert qd.cache_len() == 0
    assert qd.launch_count() == 0


@pytest.mark.parametrize("call", [
    lambda L: L.q8_0_gemv(FAKE, 33, 16, 1, FAKE, FAKE * 2, None),          # n_in % 32
    lambda L: L.q8_0_gemv(FAKE, 0, 16, 1, FAKE, FAKE * 2, None),           # n_in = 0
    lambda L: L.q8_0_gemv(FAKE, 64, -1, 1, FAKE, FAKE * 2, None),          # n_out < 0
    lambda L: L.q8_0_gemv(FAKE, 64, 16, 0, FAKE, FAKE * 2, None),          # batch 0
    lambda L: L.q8_0_gemv(FAKE, 64, 16, 9, FAKE, FAKE * 2, None),          # batch > 8
    lambda L: L.q8_0_gemv(None, 64, 16, 1, FAKE, FAKE * 2, None),          # null weight
    lambda L: L.q8_0_gemv(FAKE, 64, 16, 1, FAKE + 4, FAKE * 2, None),      # x not 16-aligned
    lambda L: L.q8_0_gemv(FAKE + 1, 64, 16, 1, FAKE, FAKE * 2, None),      # w odd address
    lambda L: L.q8_0_gemv(FAKE, 64, 16, 1, FAKE, FAKE + 16, None),         # out overlaps x
    lambda L: L.q8_0_gemv_residual(FAKE, 64, 16, 1, FAKE, None, FAKE * 2, None),
    lambda L: L.q8_0_gemv_residual(FAKE, 64, 16, 1, FAKE, FAKE * 2 + 8, FAKE * 2, None),
    lambda L: L.q8_0_qkv(FAKE, FAKE, FAKE, 64, 8, 9, 1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None),
    lambda L: L.q8_0_qkv(FAKE, FAKE, FAKE, 64, 8, 0, 1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None),
    lambda L: L.q8_0_qkv(FAKE, FAKE, FAKE, 64, 8, 4, 1, FAKE, FAKE * 2, FAKE * 2 + 16, FAKE * 4, None),
    lambda L: L.q8_0_swiglu(FAKE, None, 64, 8, 1, FAKE, FAKE * 2, None),
    lambda L: L.q4k_gemv(FAKE, 128, 8, 1, FAKE, FAKE * 2, None),           # n_in % 256
    lambda L: L.q8_0_gemm_batched(FAKE, 64, 8, 0, FAKE, FAKE * 2, None),
    lambda L: L.f32_gemm_batched(FAKE + 4, 64, 8, 1, FAKE * 4, FAKE * 8, None),
    lambda L: L.qdec_prepare(FAKE, 7, 64, 8, None),                       # unknown type
    lambda L: L.qdec_prepare(FAKE, 12, 64, 8, None),                      # Q4_K needs n_in % 256
    lambda L: L.q8_0_dequantize(FAKE, 64, 8, FAKE * 2 + 4, None),         # out not 16-aligned
    lambda L: L.qdec_copy(FAKE, FAKE * 2, 24, None),                      # bytes % 16
    lambda L: L.qdec_release(None),
    lambda L: L.qdec_attention_decode(FAKE, FAKE * 2, FAKE * 3, 24, 8, 96, 10, 100, 0.1, FAKE * 4, None),  # head_dim
    lambda L: L.qdec_attention_decode(FAKE, FAKE * 2, FAKE * 3, 24, 5, 128, 10, 100, 0.1, FAKE * 4, None),  # 5 !| 24
    lambda L: L.qdec_attention_decode(FAKE, FAKE * 2, FAKE * 3, 24, 8, 128, 101, 100, 0.1, FAKE * 4, None), # n_ctx
    lambda L: L.qdec_rope_kv_append(FAKE, FAKE * 2, FAKE * 3, 24, 8, 128, 100, 10000.0, FAKE * 4, FAKE * 5, 100, None),  # pos
    lambda L: L.q6k_gemv(FAKE, 128, 8, 1, FAKE, FAKE * 2, None),           # Q6_K needs n_in % 256
    lambda L: L.q6k_gemv(FAKE, 256, 8, 9, FAKE, FAKE * 2, None),           # batch > 8
    lambda L: L.qdec_prepare(FAKE, 14, 64, 8, None),                      # Q6_K needs n_in % 256
    lambda L: L.q6k_dequantize(FAKE, 256, 8, FAKE * 2 + 4, None),         # out not 16-aligned
    lambda L: L.q8_0_gemv_topk(FAKE, 64, 16, 1, FAKE, 0, FAKE * 2, FAKE * 3, FAKE * 4, None),    # k = 0
    lambda L: L.q8_0_gemv_topk(FAKE, 64, 16, 1, FAKE, 17, FAKE * 2, FAKE * 3, FAKE * 4, None),   # k > n_out
    lambda L: L.q8_0_gemv_topk(FAKE, 64, 400, 1, FAKE, 257, FAKE * 2, FAKE * 3, FAKE * 4, None), # k > 256
    lambda L: L.q8_0_gemv_topk(FAKE, 64, 16, 1, FAKE, 4, FAKE * 2, FAKE * 2 + 8, FAKE * 4, None),  # idx in logits
    lambda L: L.q8_0_gemv_topk(FAKE, 64, 16, 1, FAKE, 4, FAKE * 2, FAKE * 3, None, None),          # null top_val
])
def test_invalid_arguments_rejected(call):
    before = qd.launch_count()
    assert call(qd.lib) == qd.QDEC_EINVAL
    assert qd.last_error() != ""
    assert qd.launch_count() == before
    assert qd.cache_len() == 0


def test_python_wrapper_raises():
    class Fake:
        def __init__(self, p, n):
            self.p, self.n = p, n

        def data_ptr(self):
            return self.p

        def numel(self):
            return self.n

    with pytest.raises(qd.QdecError) as ei:
        qd.q8_0_gemv(Fake(FAKE, 1), 33, 4, Fake(FAKE, 33), out=Fake(FAKE * 2, 4), stream=0)
    assert ei.value.status == qd.QDEC_EINVAL
    assert "multiple of 32" in str(ei.value)


@pytest.mark.parametrize("n_in,batch,k,fits", [(3072, 8, 256, True), (3072, 5, 40, True), (3072, 3, 1, True),
                                               (1024, 8, 256, True), (8192, 8, 256, False)])
def test_noalloc_scratch_covers_the_vocabulary(n_in, batch, k, fits):
    """q8_0_gemv_topk_noalloc sizes its static scratch before anything else:
    128256 logits of n_in <= 3072 fit for every batch and k (the matrix-core
    projection's K-slice sums plus the candidate lists); 8 rows of 8192
    columns do not, and are refused by the size check itself."""
    W, X, LOG, IDX, VAL = 0x40000000, 0x1000000, 0x10000000, 0x20000000, 0x30000000
    before = qd.launch_count()
    rc = qd.lib.q8_0_gemv_topk_noalloc(W, n_in, 128256, batch, X, k, LOG, IDX, VAL, None)
    assert rc != qd.QDEC_OK          # no GPU here: a call that fits fails later, at the device
    assert ("static array" in qd.last_error()) == (not fits), qd.last_error()
    assert qd.launch_count() == before


WIDTHS = [32, 64, 96, 256, 512, 768, 1024, 1280, 2048, 2560, 3072, 4096, 6144, 7936, 8192, 8224, 16384]
ROWS = [1, 2, 15, 16, 17, 48, 77, 128, 130, 1000, 3072, 5120, 8192, 28672, 50000, 128256]
BATCHES = [1, 2, 3, 4, 5, 6, 7, 8, 9, 100, 128, 129, 512, 513]


def test_every_launch_plan_stays_in_its_buffers():
    """The host-side extent checks (the launchers run them before every
    launch) over a sweep of widths, rows and batches: every plan the library
    would choose keeps each kernel's last access inside its buffers, with the
    workspace each call would be given.  No device needed."""
    before = qd.launch_count()
    for n_in in WIDTHS:
        for n_out in ROWS:
            for batch in BATCHES:
                rc = qd.lib.qdec_check_plans(n_in, n_out, batch)
                assert rc == qd.QDEC_OK, (n_in, n_out, batch, qd.last_error())
    assert qd.lib.qdec_check_plans(33, 16, 1) == qd.QDEC_EINVAL
    assert qd.launch_count() == before
