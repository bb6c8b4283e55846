"""Pins for the CPU oracle: checks against what the definition and mathematics fix.

None of these tests compares the oracle with itself.  They use hand-built
words with literal expectations, closed forms, exact rational arithmetic,
special cases that reduce to a library routine, and invariants of the repack
permutation.  A plausible slip anywhere in the oracle (nibble order, sign of
the offset, group index, transposed operand, dropped term) fails one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_words():
    rows = []
    with open(os.path.join(GOLDEN, "unpack_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), [int(x) for x in parts[1:]]))
    return rows


# ---------------------------------------------------------------- unpack

def test_unpack_golden_words():
    rows = _golden_words()
    assert len(rows) >= 8
    qw = np.array([[w for w, _ in rows]], dtype=np.uint32)        # [1, N]
    codes = oracle.unpack(qw, 8, len(rows))                       # [8, N]
    for n, (_, expect) in enumerate(rows):
        assert codes[:, n].tolist() == expect, hex(rows[n][0])


@pytest.mark.parametrize("j", range(8))
def test_unpack_single_nibble(j):
    # word (kb=1, n=2) of a [2, 3] word array carries 0xF in nibble j only
    qw = np.zeros((2, 3), dtype=np.uint32)
    qw[1, 2] = np.uint32(0xF << (4 * j))
    codes = oracle.unpack(qw, 16, 3)
    nz = np.argwhere(codes != 0)
    assert nz.tolist() == [[8 + j, 2]]
    assert codes[8 + j, 2] == 15


def test_pack_unpack_roundtrip_all_values_all_positions():
    # every value 0..15 in every position 0..7: column v*8+p holds v at nibble p
    cols = []
    for v in range(16):
        for p in range(8):
            cols.append(v << (4 * p))
    qw = np.array([cols], dtype=np.uint32)
    codes = oracle.unpack(qw, 8, len(cols))
    for idx, (v, p) in enumerate((v, p) for v in range(16) for p in range(8)):
        expect = [0] * 8
        expect[p] = v
        assert codes[:, idx].tolist() == expect


def test_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(11)
    K, N = 64, 24
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint32)
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):                       # low nibble first
        words |= q[j::8, :] << np.uint32(4 * j)
    assert np.array_equal(oracle.unpack(words, K, N), q.astype(np.uint8))


# ---------------------------------------------------------------- bf16 reading

@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4308, 136.0), (0xC308, -136.0), (0x4300, 128.0),
    (0x3C23, 0.00994873046875), (0x0000, 0.0), (0x8000, -0.0),
    (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126), (0x7F7F, 3.3895313892515355e38),
])
def test_bf16_reading(bits, value):
    assert oracle.bf16_bits_to_f64(np.array([bits]))[0] == value
    assert oracle._bf16_fraction(bits) == Fraction(value)


def test_bf16_rne_of_fp32_exact_values():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 255.0, 257.0])
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6);
    # just above the tie rounds up; 257 = 256+1 is a tie between 256 and 258 -> 256
    expect = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x437F, 0x4380]
    assert oracle.f32_exact_to_bf16_bits(x).tolist() == expect
    with pytest.raises(ValueError):
        oracle.f32_exact_to_bf16_bits(np.array([1.0 + 2 ** -40]))


# ---------------------------------------------------------------- dequant

def _pow2_bf16(e):
    """bf16 bits of 2**e for normal exponents."""
    return ((127 + e) & 0xFF) << 7


def test_dequant_midpoint_is_zero():
    K, N = 256, 16
    qw = np.full((K // 8, N), 0x88888888, dtype=np.uint32)
    sc = np.full((K // 128, N), 0x3F80, dtype=np.uint16)
    W = oracle.dequant(qw, sc, K, N)
    assert np.all(W == 0.0)


def test_dequant_closed_form_and_group_mapping():
    # words 0xFEDCBA98 give q = 8..15, i.e. q-8 = k%8.  Scales s[g,n] = 2^(g - n%3)
    K, N = 384, 6
    qw = np.full((K // 8, N), 0xFEDCBA98, dtype=np.uint32)
    sc = np.array([[_pow2_bf16(g - n % 3) for n in range(N)] for g in range(K // 128)],
                  dtype=np.uint16)
    W = oracle.dequant(qw, sc, K, N)
    for k in (0, 1, 7, 8, 127, 128, 129, 255, 256, 383):
        for n in range(N):
            assert W[k, n] == (k % 8) * 2.0 ** (k // 128 - n % 3), (k, n)


def test_dequant_negative_codes_and_fp32_exactness():
    K, N = 128, 16
    qw = np.full((K // 8, N), 0x76543210, dtype=np.uint32)       # q-8 = k%8 - 8 in [-8, -1]
    sc = np.full((1, N), 0x4049, dtype=np.uint16)                 # 3.140625
    W = oracle.dequant(qw, sc, K, N)
    for k in range(8):
        assert W[k, 0] == (k - 8) * 3.140625
    # any (q-8)*s is exact in fp32: 8-bit significand times at most 4 bits
    A, q, s = synth.gen_problem(256, 64, seed=5)
    W = oracle.dequant(q, s, 256, 64)
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)


# ---------------------------------------------------------------- gemm

def test_gemm_against_exact_rationals():
    for seed, (M, K, N) in enumerate([(1, 128, 16), (3, 256, 8), (4, 128, 5)]):
        A, q, s = synth.gen_problem(K, N, seed=100 + seed, M=M)
        C, D = oracle.gemm(A, q, s, M, N, K)
        Ce, De = oracle.exact_gemm(A, q, s, M, N, K)
        for m in range(M):
            for n in range(N):
                bound = K * 2.0 ** -53 * float(De[m][n])
                assert abs(Fraction(C[m, n]) - Ce[m][n]) <= Fraction(bound)
                assert abs(Fraction(D[m, n]) - De[m][n]) <= Fraction(bound)


@pytest.mark.parametrize("word,colsum,abssum", [
    (0x76543210, -36, 36),      # q-8 = -8..-1 per word
    (0xFEDCBA98, 28, 28),       # q-8 = 0..7
    (0xFFFFFFFF, 56, 56),       # 8 * 7
    (0x00000000, -64, 64),      # 8 * -8
    (0x88888888, 0, 0),
])
def test_gemm_ones_closed_form(word, colsum, abssum):
    # A = ones, s = 2^-3: C[n] = 2^-3 * (K/8) * colsum(word); exact
    M, K, N = 2, 512, 16
    A = np.full((M, K), 0x3F80, dtype=np.uint16)
    qw = np.full((K // 8, N), word, dtype=np.uint32)
    sc = np.full((K // 128, N), _pow2_bf16(-3), dtype=np.uint16)
    C, D = oracle.gemm(A, qw, sc, M, N, K)
    assert np.all(C == colsum * (K // 8) * 2.0 ** -3)
    assert np.all(D == abssum * (K // 8) * 2.0 ** -3)


def test_gemm_one_hot_picks_row_and_group():
    # q-8 = k%8 (word 0xFEDCBA98), s[g, n] = 2^(g - n%3); A row m = one-hot at k_m
    K, N = 384, 7
    qw = np.full((K // 8, N), 0xFEDCBA98, dtype=np.uint32)
    sc = np.array([[_pow2_bf16(g - n % 3) for n in range(N)] for g in range(K // 128)],
                  dtype=np.uint16)
    ks = [5, 127, 128, 263]
    A = np.zeros((len(ks), K), dtype=np.uint16)
    for m, k in enumerate(ks):
        A[m, k] = 0x3F80
    C, D = oracle.gemm(A, qw, sc, len(ks), N, K)
    for m, k in enumerate(ks):
        for n in range(N):
            assert C[m, n] == (k % 8) * 2.0 ** (k // 128 - n % 3), (m, n)
            assert D[m, n] == abs(C[m, n])


def test_gemm_distinguishes_rows_and_columns():
    # A non-square, asymmetric case: a transposed operand or swapped index fails
    K, N = 256, 3
    qw = np.zeros((K // 8, N), dtype=np.uint32)
    qw[:, 0] = 0xFFFFFFFF          # column 0: q-8 = 7
    qw[:, 1] = 0x88888888          # column 1: q-8 = 0
    qw[:, 2] = 0x00000000          # column 2: q-8 = -8
    sc = np.full((2, N), 0x3F80, dtype=np.uint16)
    A = np.zeros((2, K), dtype=np.uint16)
    A[0, :] = 0x3F80               # row 0: all ones
    A[1, 0] = 0x4000               # row 1: 2.0 at k=0 only
    C, _ = oracle.gemm(A, qw, sc, 2, N, K)
    assert C.tolist() == [[7.0 * K, 0.0, -8.0 * K], [14.0, 0.0, -16.0]]


def test_gemm_matches_numpy_matmul_on_dequantized_matrix():
    M, K, N = 5, 640, 48
    A, q, s = synth.gen_problem(K, N, seed=7, M=M)
    W = oracle.dequant(q, s, K, N)
    Af = oracle.bf16_bits_to_f64(A)
    ref = Af @ W
    C, D = oracle.gemm(A, q, s, M, N, K)
    bound = 1e-12 * (np.abs(Af) @ np.abs(W))
    assert np.all(np.abs(C - ref) <= bound)
    assert np.allclose(D, np.abs(Af) @ np.abs(W), rtol=1e-13)


def test_gemm_column_subset_and_thread_count_invariance():
    M, K, N = 3, 512, 64
    A, q, s = synth.gen_problem(K, N, seed=8, M=M)
    C, D = oracle.gemm(A, q, s, M, N, K, nthreads=1)
    C4, D4 = oracle.gemm(A, q, s, M, N, K, nthreads=4)
    assert np.array_equal(C, C4) and np.array_equal(D, D4)
    cols = [63, 0, 17, 17, 40]
    Cs, Ds = oracle.gemm(A, q, s, M, N, K, cols=cols)
    assert np.array_equal(Cs, C[:, cols]) and np.array_equal(Ds, D[:, cols])


# ---------------------------------------------------------------- repack

def test_repack_literal_positions():
    # K=256 (G=2), N=32 (2 tiles).  Word index = piece*4 + r with
    # piece = ((t*G + g)*4 + h)*16 + c; even row offset e -> bit 4*(e/2), odd -> 16 + 4*(e/2)
    K, N = 256, 32
    cases = [  # (k, n, word index, bit)
        (0, 0, 0, 0), (1, 0, 0, 16), (2, 0, 0, 4), (7, 0, 0, 28), (6, 0, 0, 12),
        (8, 0, 1, 0), (31, 0, 3, 28), (32, 0, 64, 0), (128, 0, 256, 0),
        (0, 1, 4, 0), (0, 15, 60, 0), (0, 16, 512, 0), (255, 31, 1023, 28),
        (133, 20, 512 + 256 + 16 + 0 + 0 * 4 + 0, 0),
    ]
    # (133, 20): t=1, c=4, g=1, h=0, r=0, e=5 -> piece ((1*2+1)*4+0)*16+4 = 196,
    # word 784, bit 16 + 4*2 = 24
    cases[-1] = (133, 20, 784, 24)
    for k, n, widx, bit in cases:
        qw = np.zeros((K // 8, N), dtype=np.uint32)
        qw[k // 8, n] = np.uint32(0x9 << (4 * (k % 8)))
        blob = oracle.repack(qw, K, N)
        nz = np.nonzero(blob)[0].tolist()
        assert nz == [widx], (k, n, nz)
        assert int(blob[widx]) == 0x9 << bit, (k, n, hex(int(blob[widx])))


def test_repack_is_a_bijection_preserving_nibbles():
    for K, N in [(128, 16), (384, 48), (512, 1024)]:
        _, q, _ = synth.gen_problem(K, N, seed=K + N, M=1)
        blob = oracle.repack(q, K, N)
        assert blob.size == K * N // 8
        assert np.array_equal(oracle.unrepack(blob, K, N), q)
        hist_q = np.bincount(oracle.unpack(q, K, N).ravel(), minlength=16)
        nib = np.stack([(blob >> np.uint32(4 * j)) & np.uint32(0xF) for j in range(8)])
        hist_b = np.bincount(nib.ravel().astype(np.int64), minlength=16)
        assert np.array_equal(hist_q, hist_b)


# ---------------------------------------------------------------- metric

def test_normalized_error():
    C_ref = np.array([[1.0, 0.0, -2.0]])
    D_ref = np.array([[4.0, 0.0, 8.0]])
    e = oracle.normalized_error(np.array([[1.5, 0.0, -2.0]]), C_ref, D_ref)
    assert e.tolist() == [[0.125, 0.0, 0.0]]
    e = oracle.normalized_error(np.array([[1.0, -0.0, -2.0]]), C_ref, D_ref)
    assert e.tolist() == [[0.0, 0.0, 0.0]]
    e = oracle.normalized_error(np.array([[1.0, 1e-30, -2.0]]), C_ref, D_ref)
    assert np.isinf(e[0, 1])


# ---------------------------------------------------------------- geometry

def test_geometry_matches_kv_cache_figure():
    # Page "One Config Line Made My 27B Model 2.7x Faster", section "The machine
    # and the model": only the 16 full-attention layers keep a KV cache, about
    # 64 KiB per token, about 8.6 GB at a 128K context.  With 4 KV heads of
    # head_dim 256 in bf16 (page "Qwen3.8 27B - NVFP4 for veloGB10",
    # "Specifications"), K and V per layer per token:
    kv_bytes = 16 * 2 * 4 * 256 * 2
    assert kv_bytes == 64 * 1024
    assert round(131072 * kv_bytes / 1e9, 1) == 8.6
    # the same heads give the QKV-shaped workload's N: 24 Q heads + 2 x 4 KV heads
    assert (24 + 2 * 4) * 256 == synth.WORKLOADS["qkv"].N
    assert 2 * 17408 == synth.WORKLOADS["gate_up"].N
    assert synth.WORKLOADS["lm_head"].N == 248320


# ----------------------------------------------------------------- gate/up activation

def test_silu_closed_forms_and_identity():
    # silu(x) - silu(-x) = x (x s(x) + x s(-x) = x since s(x) + s(-x) = 1)
    x = np.linspace(-30.0, 30.0, 241)
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-12)
    # s(ln 3) = 3/4 exactly in the reals
    assert abs(oracle.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # no overflow at finite extremes
    big = oracle.silu(np.array([-1e6, 1e6, -700.0, 700.0]))
    assert big[0] == 0.0 and big[1] == 1e6 and abs(big[2]) < 1e-290 and big[3] == 700.0
    # derivative against a central difference
    h = 1e-6
    xs = np.array([-5.0, -1.0, 0.0, 0.5, 3.0])
    num = (oracle.silu(xs + h) - oracle.silu(xs - h)) / (2 * h)
    assert np.allclose(oracle.silu_derivative(xs), num, rtol=0, atol=1e-8)


def test_gemm_silu_mul_halves_are_gate_then_up():
    # one-hot A on row k, scales 1: C[0, n] = q[k, n] - 8 exactly, so
    # H[0, j] = silu(q[k, j] - 8) * (q[k, j + N/2] - 8)
    K, N, k = 256, 64, 131
    rng = np.random.default_rng(5)
    qw = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint32)
    sc = np.full((K // 128, N), 0x3F80, dtype=np.uint16)            # 1.0
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, k] = 0x3F80
    H, E = oracle.gemm_silu_mul(A, qw, sc, 1, N, K)
    q = oracle.unpack(qw, K, N)[k].astype(np.int64) - 8
    for j in range(N // 2):
        g, u = float(q[j]), float(q[j + N // 2])
        want = g / (1.0 + math.exp(-g)) * u
        assert abs(H[0, j] - want) <= 1e-12 * max(1.0, abs(want)), (j, H[0, j], want)
    # zero gate codes (8) give exact zeros whatever the up half holds, and
    # not the other way round
    qw_gate0 = qw.copy()
    qw_gate0[:, : N // 2] = 0x88888888
    H0, E0 = oracle.gemm_silu_mul(A, qw_gate0, sc, 1, N, K)
    assert np.all(H0 == 0.0)
    qw_up0 = qw.copy()
    qw_up0[:, N // 2:] = 0x88888888
    H1, _ = oracle.gemm_silu_mul(A, qw_up0, sc, 1, N, K)
    assert np.all(H1 == 0.0)
    qw_swapped = np.concatenate([qw[:, N // 2:], qw[:, : N // 2]], axis=1)
    Hs, _ = oracle.gemm_silu_mul(A, qw_swapped, sc, 1, N, K)
    assert not np.allclose(Hs, H)


def test_gemm_silu_mul_column_subset_and_bound():
    K, N = 384, 96
    A, qw, sc = synth.gen_problem(K, N, 12)
    H, E = oracle.gemm_silu_mul(A, qw, sc, 3, N, K)
    js = np.array([0, 7, 47, 20])
    Hs, Es = oracle.gemm_silu_mul(A, qw, sc, 3, N, K, js=js)
    assert np.array_equal(Hs, H[:, js]) and np.array_equal(Es, E[:, js])
    assert np.all(E >= 0)
    # moving g and u by at most 1e-6 of their D changes H by at most about 1e-6 E
    C, D = oracle.gemm(A, qw, sc, 3, N, K)
    g, u = C[:, : N // 2], C[:, N // 2:]
    dg, du = D[:, : N // 2], D[:, N // 2:]
    eps = 1e-6
    H2 = oracle.silu(g + eps * dg) * (u - eps * du)
    assert np.all(np.abs(H2 - H) <= eps * E * 1.01 + 1e-15)


# ----------------------------------------------------------------- greedy pick

def test_row_argmax_ties_and_signed_zero():
    C = np.array([[1.0, 3.0, 3.0, 2.0],
                  [-0.0, 0.0, -1.0, -0.0],
                  [-5.0, -4.0, -4.0, -7.0],
                  [np.nan, 1.0, 2.0, 0.5]])
    got = oracle.row_argmax(C)
    assert got[0] == 1          # lowest of the equal maxima
    assert got[1] == 0          # -0 == +0: the first of them
    assert got[2] == 1
    assert got.dtype.kind == "i"
    # on the gemm: a one-hot A picks row k of W, so the argmax is the column
    # of the largest (q - 8) * s in that row
    K, N, k = 256, 48, 77
    rng = np.random.default_rng(9)
    qw = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint32)
    sc = oracle.f32_exact_to_bf16_bits(np.abs(rng.standard_normal((K // 128, N))).astype(np.float32))
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, k] = 0x3F80
    C, _ = oracle.gemm(A, qw, sc, 1, N, K)
    W = oracle.dequant(qw, sc, K, N)
    assert oracle.row_argmax(C)[0] == int(np.argmax(W[k]))
