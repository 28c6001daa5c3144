"""Input generators (no GPU): the recipes' fixed points and the log
fingerprint."""
import numpy as np

import synth

PRIME = 0x100000001B3
MASK = (1 << 64) - 1


def test_fnv1a_published_vectors():
    """The byte loop against the FNV-1a 64-bit test vectors of the hash's
    published definition ("" -> offset basis, "a", "foobar"); with n_in =
    n_out = 0 the two trailing folds are two multiplications by the prime."""
    for data, h in ((b"", 0xCBF29CE484222325), (b"a", 0xAF63DC4C8601EC8C), (b"foobar", 0x85944171F73967E8)):
        want = (h * PRIME * PRIME) & MASK
        arr = np.frombuffer(data, np.uint8)
        assert synth.fnv1a64_py(arr, 0, 0) == want
        assert synth.fnv1a64(arr, 0, 0) == want


def test_fnv1a_compiled_matches_python_and_folds_dims():
    rng = np.random.default_rng(5)
    raw = rng.integers(0, 256, 5000, dtype=np.uint8)
    for n_in, n_out in ((3072, 8192), (32, 1), (2 ** 40 + 3, 7)):
        assert synth.fnv1a64(raw, n_in, n_out) == synth.fnv1a64_py(raw, n_in, n_out)
    # the dims are part of the key: a transposed shape has another fingerprint
    assert synth.fnv1a64(raw, 3072, 8192) != synth.fnv1a64(raw, 8192, 3072)


def test_q8_0_generator_fixed_points():
    """d = amax/127 stored as fp16, q = round-half-away(w/d) within [-127, 127]."""
    raw, w = synth.q8_0_weights(9, 4, 64)
    blk = raw.reshape(4, 2, 34)
    d = blk[:, :, 0:2].copy().view(np.float16).reshape(4, 2).astype(np.float32)
    q = blk[:, :, 2:].view(np.int8).astype(np.int32)
    amax = np.abs(w.reshape(4, 2, 32)).max(axis=2)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float16).astype(np.float32))
    assert np.abs(q).max() <= 127 and (np.abs(q).max(axis=2) == 127).all()
