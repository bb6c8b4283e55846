"""Pins of the NVFP4 oracle (oracle/nvfp4.c) against what the formats and the
mathematics fix, never against a re-typing of its own formula.

  * E2M1 and E4M3 values: literal tables of the published formats
    (tests/golden/), and for E4M3 also torch's float8_e4m3fn conversion (an
    independent library route) over all 256 bytes;
  * unpack: literal bytes with known nibbles;
  * repack: literal positions, a byte permutation, round trip;
  * GEMM: exact rational brute force, one-hot and all-ones closed forms built
    from the golden tables, a numpy matmul route, per-tensor factor scaling,
    and the 16-row scale-block boundary.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split()
        out[int(key, 16)] = float(val)
    return out


E2M1 = _table("nvfp4_e2m1.txt")
E4M3 = _table("e4m3_values.txt")


def _same(a, b):
    """Equal values with equal signs (so -0 != +0), NaN equal to NaN."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_golden_table():
    assert len(E2M1) == 16
    got = oracle.e2m1_to_f64(np.arange(16))
    for code, val in E2M1.items():
        assert _same(got[code], val), (code, got[code], val)
    # sign bit: code ^ 8 is the negation; positive codes are increasing
    assert all(_same(got[c ^ 8], -got[c]) for c in range(16))
    assert np.all(np.diff(got[:8]) > 0)


def test_e4m3_golden_values_and_library_route():
    import torch
    got = oracle.e4m3_to_f64(np.arange(256))
    for b, val in E4M3.items():
        assert _same(got[b], val), (hex(b), got[b], val)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        assert _same(got[b], float(lib[b])), (hex(b), got[b], lib[b])
    finite = got[~np.isnan(got)]
    assert finite.max() == 448.0 and np.sum(np.isnan(got)) == 2


def test_nvfp4_unpack_literal_bytes():
    K, N = 16, 3
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    packed[0, 0] = 0x21          # k=0 -> 1, k=1 -> 2
    packed[1, 7] = 0xF0          # k=14 -> 0, k=15 -> 15
    packed[2, 3] = 0x8C          # k=6 -> 12, k=7 -> 8
    codes = oracle.nvfp4_unpack(packed, K, N)
    assert codes.shape == (K, N)
    want = np.zeros((K, N), dtype=np.uint8)
    want[0, 0], want[1, 0] = 1, 2
    want[14, 1], want[15, 1] = 0, 15
    want[6, 2], want[7, 2] = 12, 8
    assert np.array_equal(codes, want)


@pytest.mark.parametrize("k,n,byte,high", [
    (0, 0, 0, False), (1, 0, 0, True), (2, 0, 1, False), (3, 0, 1, True),
    (4, 0, 256, False),                      # rows 4..7 of a block: lane group h = 1 (piece 16)
    (12, 0, 768, False),                     # h = 3 (piece 48)
    (16, 0, 2, False),                       # next 16-row block: byte 2 of the piece
    (127, 0, 3 * 256 + 15, True),            # last row of the superblock: b = 7, h = 3, p = 1
    (128, 0, 1024, False),                   # next superblock: next 1 KiB
    (0, 1, 16, False),                       # next column: next piece
    (0, 17, ((1 * 2 + 0) * 4 + 0) * 16 * 16 + 16, False),   # tile 1, column 1
    (133, 18, (((1 * 2 + 1) * 4 + 1) * 16 + 2) * 16 + 0, True),
])
def test_nvfp4_repack_literal_positions(k, n, byte, high):
    K, N = 256, 32
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    packed[n, k // 2] = 0x5 << (4 * (k % 2))
    blob = oracle.nvfp4_repack(packed, K, N)
    nz = np.nonzero(blob)[0]
    assert nz.tolist() == [byte]
    assert blob[byte] == (0x50 if high else 0x05)


def test_nvfp4_repack_is_a_byte_permutation_and_inverts():
    K, N = 384, 48
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    blob = oracle.nvfp4_repack(packed, K, N)
    assert blob.size == K * N // 2
    assert np.array_equal(np.sort(blob), np.sort(packed.ravel()))
    assert np.array_equal(oracle.nvfp4_unrepack(blob, K, N), packed)


def test_nvfp4_repack_scales_literal_positions_and_permutation():
    K, N = 256, 32
    sc = np.zeros((N, K // 16), dtype=np.uint8)
    sc[17, 9] = 0x38             # column 17 = tile 1, c 1; block 9 = superblock 1, b 1
    out = oracle.nvfp4_repack_scales(sc, K, N)
    assert np.nonzero(out)[0].tolist() == [((1 * 2 + 1) * 16 + 1) * 8 + 1]
    rng = np.random.default_rng(4)
    sc = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    out = oracle.nvfp4_repack_scales(sc, K, N)
    assert np.array_equal(np.sort(out), np.sort(sc.ravel()))
    # a column's 8 block scales of one superblock are one run of 8 bytes
    t, c, g = 1, 5, 1
    base = ((t * 2 + g) * 16 + c) * 8
    assert np.array_equal(out[base:base + 8], sc[16 * t + c, 8 * g:8 * g + 8])


def _f32(x):
    return float(np.float32(x))


@pytest.mark.parametrize("M,K,N,seed", [(1, 128, 16, 0), (3, 128, 32, 1), (2, 256, 16, 2)])
def test_nvfp4_gemm_against_exact_rationals(M, K, N, seed):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    # every finite byte, subnormal and negative scales included
    scales = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x38
    A = synth.gen_activations(M, K, rng)
    alpha = _f32(0.0037)
    C, D = oracle.nvfp4_gemm(A, packed, scales, alpha, M, N, K)
    ex = oracle.nvfp4_exact_gemm(A, packed, scales, Fraction(alpha), M, N, K)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(C[m, n]) - ex[m][n]) <= Fraction(K) * Fraction(2) ** -53 * Fraction(D[m, n]), (m, n)


def test_nvfp4_gemm_one_hot_picks_element_scale_and_block():
    # one-hot A on row k and alpha 1: C[0, n] = e2m1(code(k, n)) * e4m3(scale(k // 16, n))
    K, N = 256, 32
    rng = np.random.default_rng(6)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    # distinct scale per (column, block): E4M3 powers of two 2^(e-7), e = 1..14
    e = (np.arange(N)[:, None] + np.arange(K // 16)[None, :]) % 14 + 1
    scales = (e << 3).astype(np.uint8)
    for k in (0, 1, 15, 16, 17, 127, 128, 255):
        A = np.zeros((1, K), dtype=np.uint16)
        A[0, k] = 0x3F80
        C, D = oracle.nvfp4_gemm(A, packed, scales, 1.0, 1, N, K)
        for n in range(N):
            byte = int(packed[n, k // 2])
            code = byte & 0xF if k % 2 == 0 else byte >> 4
            want = E2M1[code] * 2.0 ** (int(e[n, k // 16]) - 7)
            assert C[0, n] == want and D[0, n] == abs(want), (k, n, C[0, n], want)


def test_nvfp4_gemm_ones_column_sums_from_the_table():
    # A = 1, scales 1.0 (0x38), alpha 1: C[m, n] = sum over k of the E2M1 values of column n
    K, N = 256, 16
    rng = np.random.default_rng(7)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x38, dtype=np.uint8)
    A = np.full((2, K), 0x3F80, dtype=np.uint16)
    C, _ = oracle.nvfp4_gemm(A, packed, scales, 1.0, 2, N, K)
    for n in range(N):
        want = sum(E2M1[int(b) & 0xF] + E2M1[int(b) >> 4] for b in packed[n])
        assert C[0, n] == want and C[1, n] == want


def test_nvfp4_gemm_matches_numpy_on_dequantized_matrix_and_alpha_scales():
    K, N, M = 384, 48, 4
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 8, M=M)
    W = oracle.nvfp4_dequant(packed, scales, K, N)
    a = oracle.bf16_bits_to_f64(A[:M])
    C1, D1 = oracle.nvfp4_gemm(A, packed, scales, 1.0, M, N, K)
    assert np.allclose(C1, a @ W, rtol=0, atol=1e-12 * D1.max())
    assert np.allclose(D1, np.abs(a) @ np.abs(W), rtol=1e-14)
    # a power-of-two factor scales exactly; a negative one flips the sign, not D
    C2, D2 = oracle.nvfp4_gemm(A, packed, scales, -2.0 ** -5, M, N, K)
    assert np.array_equal(C2, -(2.0 ** -5) * C1) and np.array_equal(D2, 2.0 ** -5 * D1)
    # column subsets equal the full result
    cols = np.array([47, 0, 16, 3])
    Cs, Ds = oracle.nvfp4_gemm(A, packed, scales, 1.0, M, N, K, cols=cols)
    assert np.array_equal(Cs, C1[:, cols]) and np.array_equal(Ds, D1[:, cols])


def test_nvfp4_dequant_products_are_fp32_exact():
    # e2m1 (2 significant bits) times e4m3 (4 bits) fits fp32 exactly,
    # subnormal scales included: the device export can be compared bitwise
    K, N = 128, 16
    rng = np.random.default_rng(9)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x01
    W = oracle.nvfp4_dequant(packed, scales, K, N)
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)


def test_nvfp4_gemm_silu_mul_halves_alpha_and_zero_gate():
    # one-hot A on row k, scales 1.0 (0x38): C[0, n] = alpha * e2m1(code(k, n)), so
    # H[0, j] = silu(alpha g_j) * alpha u_j with g, u read from the table
    K, N, k = 256, 64, 77
    rng = np.random.default_rng(11)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x38, dtype=np.uint8)
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, k] = 0x3F80
    codes = packed[:, k // 2] >> 4 if k % 2 else packed[:, k // 2] & 0xF
    for alpha in (1.0, 0.5, -2.0):
        H, E = oracle.nvfp4_gemm_silu_mul(A, packed, scales, alpha, 1, N, K)
        for j in range(N // 2):
            g = alpha * E2M1[int(codes[j])]
            u = alpha * E2M1[int(codes[j + N // 2])]
            want = g / (1.0 + math.exp(-g)) * u
            assert abs(H[0, j] - want) <= 1e-12 * max(1.0, abs(want)), (alpha, j, H[0, j], want)
        assert np.all(E >= 0)
    # gate codes 0 (+0) and 8 (-0) give exact zeros whatever the up half holds
    p0 = packed.copy()
    p0[: N // 2] = np.where(rng.integers(0, 2, size=p0[: N // 2].shape) > 0, 0x00, 0x88).astype(np.uint8)
    A2 = synth.gen_activations(3, K, rng)
    H0, _ = oracle.nvfp4_gemm_silu_mul(A2, p0, scales, 0.25, 3, N, K)
    assert np.all(H0 == 0.0)
    # column subsets equal the full result
    H, E = oracle.nvfp4_gemm_silu_mul(A2, packed, scales, 0.25, 3, N, K)
    js = np.array([31, 0, 9])
    Hs, Es = oracle.nvfp4_gemm_silu_mul(A2, packed, scales, 0.25, 3, N, K, js=js)
    assert np.array_equal(Hs, H[:, js]) and np.array_equal(Es, E[:, js])


def test_nvfp4_row_argmax_follows_the_sign_of_alpha():
    # one-hot A picks row k of W: the argmax of alpha * W[k] is the column of
    # the largest entry for alpha > 0 and of the smallest for alpha < 0
    K, N, k = 128, 48, 40
    rng = np.random.default_rng(12)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0x30, 0x50, size=(N, K // 16), dtype=np.uint8)
    A = np.zeros((1, K), dtype=np.uint16)
    A[0, k] = 0x3F80
    W = oracle.nvfp4_dequant(packed, scales, K, N)
    Cp, _ = oracle.nvfp4_gemm(A, packed, scales, 0.5, 1, N, K)
    Cn, _ = oracle.nvfp4_gemm(A, packed, scales, -0.5, 1, N, K)
    assert oracle.row_argmax(Cp)[0] == int(np.argmax(W[k]))
    assert oracle.row_argmax(Cn)[0] == int(np.argmin(W[k]))
