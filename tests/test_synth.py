"""The seeded generators: determinism, shapes and distributions."""
import numpy as np

import oracle
import synth


def test_same_seed_same_bytes_and_draw_order():
    a1 = synth.gen_problem(512, 64, seed=3)
    a2 = synth.gen_problem(512, 64, seed=3)
    for x, y in zip(a1, a2):
        assert x.tobytes() == y.tobytes()
    b = synth.gen_problem(512, 64, seed=4)
    assert a1[1].tobytes() != b[1].tobytes()
    # the first M rows of A do not depend on how many rows are drawn after them
    A4, _, _ = synth.gen_problem(512, 64, seed=3, M=4)
    assert np.array_equal(A4, a1[0][:4])


def test_shapes_and_distributions():
    K, N = 1024, 2048
    A, q, s = synth.gen_problem(K, N, seed=0)
    assert A.shape == (16, K) and A.dtype == np.uint16
    assert q.shape == (K // 8, N) and q.dtype == np.uint32
    assert s.shape == (K // 128, N) and s.dtype == np.uint16
    codes = oracle.unpack(q, K, N)
    hist = np.bincount(codes.ravel(), minlength=16) / codes.size
    assert np.all(np.abs(hist - 1 / 16) < 0.003)
    sv = oracle.bf16_bits_to_f64(s)
    assert np.all(sv >= 0) and abs(sv.mean() - 0.01 * np.sqrt(2 / np.pi)) < 2e-4
    av = oracle.bf16_bits_to_f64(A)
    assert abs(av.mean()) < 0.02 and abs(av.std() - 1) < 0.02


def test_silu_mul_activations():
    A = synth.gen_activations(16, 4096, np.random.default_rng(1), "silu_mul")
    av = oracle.bf16_bits_to_f64(A)
    # E[SiLU(x) y] = 0 and the distribution is heavy on small values
    assert abs(av.mean()) < 0.02
    assert 0.4 < av.std() < 0.8


def test_algorithmic_bytes():
    # K*N/2 + (K/128)*N*2 + M*K*2 + M*N*2
    assert synth.algorithmic_bytes(1, 8192, 5120) == 20971520 + 655360 + 10240 + 16384
    assert synth.algorithmic_bytes(16, 248320, 5120) == 635699200 + 19865600 + 163840 + 7946240


def test_nvfp4_inputs_documented_ranges_and_order():
    K, N = 512, 64
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 5)
    assert packed.shape == (N, K // 2) and packed.dtype == np.uint8
    assert scales.shape == (N, K // 16) and scales.dtype == np.uint8
    # every code value appears (uniform bytes hold two uniform nibbles)
    assert set(np.unique(packed & 0xF)) == set(range(16))
    assert set(np.unique(packed >> 4)) == set(range(16))
    # E4M3 scales: sign 0, exponent field 4..10, any mantissa; never NaN
    e = (scales >> 3) & 0xF
    assert np.all(scales < 0x80) and e.min() >= 4 and e.max() <= 10
    assert not np.any((scales & 0x7F) == 0x7F)
    # draw order: codes, scales, then A from the same generator
    rng = np.random.default_rng(5)
    p2, s2 = synth.gen_nvfp4_weights(K, N, rng)
    A2 = synth.gen_activations(16, K, rng)
    assert np.array_equal(p2, packed) and np.array_equal(s2, scales) and np.array_equal(A2, A)
    assert synth.NVFP4_ALPHA == float(np.float32(0.0037))
    assert synth.algorithmic_bytes_nvfp4(1, 8192, 5120) == 5120 * 8192 // 2 + 320 * 8192 + 5120 * 2 + 8192 * 2
