"""CPU tests of the seeded input generators."""
import hashlib

import numpy as np

from rank_linear_layer_amd import datagen


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_deterministic_and_seed_sensitive():
    a = datagen.factorized_inputs(4, 64, 13, 32, 123)
    b = datagen.factorized_inputs(4, 64, 13, 32, 123)
    c = datagen.factorized_inputs(4, 64, 13, 32, 124)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and _h(x) == _h(y)
    assert _h(a[0]) != _h(c[0])


def test_bf16_round_to_nearest_even():
    f = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0xBF808000,
                  0x00000000, 0x80000000, 0x3F800000], dtype=np.uint32).view(np.float32)
    got = datagen.bf16_bits_from_f32(f)
    want = np.array([0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF80, 0x0000, 0x8000, 0x3F80], dtype=np.uint16)
    assert np.array_equal(got, want)
    # round trip of representable values is exact
    bits = np.array([0x3F80, 0x4049, 0xC2F7, 0x0001, 0x7F7F], dtype=np.uint16)
    assert np.array_equal(datagen.bf16_bits_from_f32(datagen.bf16_bits_to_f32(bits)), bits)


def test_distribution_scales():
    X, A, B = datagen.factorized_inputs(64, 1024, 256, 512, 9)
    x = datagen.bf16_bits_to_f32(X)
    a = datagen.bf16_bits_to_f32(A)
    b = datagen.bf16_bits_to_f32(B)
    assert abs(x.std() - 1.0) < 0.02
    assert abs(a.std() * np.sqrt(1024) - 1.0) < 0.02
    assert abs(b.std() * np.sqrt(256) - 1.0) < 0.02
    assert abs(x.mean()) < 0.02


def test_svd_factor_inputs_shapes():
    W, A64, B64, Ab, Bb = datagen.svd_factor_inputs(64, 48, 5, 1)
    assert W.shape == (64, 48) and A64.shape == (64, 5) and B64.shape == (5, 48)
    assert Ab.shape == (64, 5) and Bb.shape == (5, 48) and Ab.dtype == np.uint16
