"""CPU oracle for the W4A16 decode/verify matmul.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and the two share no code: the only thing
both sides consume is the seeded input generator in ``synth.py``, which holds
none of the method's arithmetic.

Contents
  * ``unpack``, ``dequant``, ``gemm``, ``repack``, ``unrepack``: thin numpy
    wrappers around ``oracle.c`` (fp64, plain loops), built with gcc into
    ``liboracle.so`` next to this file.
  * ``exact_gemm``: exact rational arithmetic (Python ``Fraction``) for tiny
    shapes, used to pin the fp64 oracle.
  * ``normalized_error``: the acceptance metric
    ``max |C_gpu - C_ref| / sum|a*w|`` per output.
  * ``bf16_bits_to_f64`` / ``f32_exact_to_bf16_bits``: exact bf16 reading,
    and round-to-nearest-even of fp32-representable values to bf16.
  * ``silu``, ``gemm_silu_mul``, ``row_argmax``: the gate/up activation and
    the greedy pick on top of ``gemm``.
  * ``nvfp4_*``: the NVFP4 weight-only variant (E2M1 codes, one E4M3 scale
    per 16 rows, an fp32 per-tensor factor), wrappers around ``nvfp4.c``;
    ``nvfp4_exact_gemm`` in exact rationals for tiny shapes.

What is computed follows the checkpoint contract on the page "Qwen3.8-27B on
single DGX Spark ..." (section "Quality."): symmetric GPTQ, 4-bit, group 128,
BF16 activations, no act-order, no zero points, with the runtime judged
against exact dequantization of its checkpoint.  The oracle is that exact
dequantization followed by an fp64 dot product.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

GROUP = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "oracle.c"), os.path.join(_HERE, "nvfp4.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c and nvfp4.c with gcc (portable x86-64, OpenMP) into liboracle.so."""
    stale = os.path.exists(_LIB_PATH) and any(os.path.getmtime(s) > os.path.getmtime(_LIB_PATH) for s in _SRCS)
    if force or stale or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, *_SRCS, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_unpack.argtypes = [P, i, i, P]
        lib.oracle_dequant.argtypes = [P, P, i, i, P]
        lib.oracle_gemm.argtypes = [P, P, P, i, i, i, P, i, i, P, P]
        lib.oracle_repack.argtypes = [P, i, i, P]
        lib.oracle_unrepack.argtypes = [P, i, i, P]
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_max_threads.restype = ctypes.c_int
        d = ctypes.c_double
        lib.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint]
        lib.oracle_e2m1_to_f64.restype = d
        lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint]
        lib.oracle_e4m3_to_f64.restype = d
        lib.oracle_nvfp4_unpack.argtypes = [P, i, i, P]
        lib.oracle_nvfp4_dequant.argtypes = [P, P, i, i, P]
        lib.oracle_nvfp4_gemm.argtypes = [P, P, P, d, i, i, i, P, i, i, P, P]
        lib.oracle_nvfp4_repack.argtypes = [P, i, i, P]
        lib.oracle_nvfp4_unrepack.argtypes = [P, i, i, P]
        lib.oracle_nvfp4_repack_scales.argtypes = [P, i, i, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_shapes(K: int, N: int, multiple: int = GROUP):
    if K % multiple or K <= 0 or N <= 0:
        raise ValueError(f"oracle: K must be a positive multiple of {multiple}, N positive")


def unpack(qweight: np.ndarray, K: int, N: int) -> np.ndarray:
    """Codes q[k, n] in [0, 15] from GPTQ words uint32 [K/8, N] (low nibble first)."""
    _check_shapes(K, N, 8)
    qw = np.ascontiguousarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    out = np.empty((K, N), dtype=np.uint8)
    _load().oracle_unpack(_ptr(qw), K, N, _ptr(out))
    return out


def dequant(qweight: np.ndarray, scales: np.ndarray, K: int, N: int) -> np.ndarray:
    """W[k, n] = (q - 8) * s[k // 128, n] in fp64 (exactly fp32-representable)."""
    _check_shapes(K, N)
    qw = np.ascontiguousarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    sc = np.ascontiguousarray(scales, dtype=np.uint16).reshape(K // GROUP, N)
    out = np.empty((K, N), dtype=np.float64)
    _load().oracle_dequant(_ptr(qw), _ptr(sc), K, N, _ptr(out))
    return out


def gemm(A: np.ndarray, qweight: np.ndarray, scales: np.ndarray, M: int, N: int, K: int,
         cols=None, nthreads: int = 0):
    """fp64 reference C[M, ncols] = A . dequant(W)[:, cols] and D = sum |a*w|.

    ``A`` is bf16 bits (uint16) [M, K]; ``cols`` selects output columns (all if None).
    Returns (C, D), both float64 [M, ncols].
    """
    _check_shapes(K, N)
    if not 1 <= M <= 16:
        raise ValueError("oracle.gemm: 1 <= M <= 16")
    a = np.ascontiguousarray(A, dtype=np.uint16).reshape(-1, K)[:M]
    a = np.ascontiguousarray(a)
    qw = np.ascontiguousarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    sc = np.ascontiguousarray(scales, dtype=np.uint16).reshape(K // GROUP, N)
    if cols is None:
        ncols = N
        cptr = None
    else:
        c = np.ascontiguousarray(cols, dtype=np.int32)
        if c.size and (c.min() < 0 or c.max() >= N):
            raise ValueError("oracle.gemm: column index out of range")
        ncols = int(c.size)
        cptr = _ptr(c)
    C = np.empty((M, ncols), dtype=np.float64)
    D = np.empty((M, ncols), dtype=np.float64)
    _load().oracle_gemm(_ptr(a), _ptr(qw), _ptr(sc), M, N, K, cptr, ncols, int(nthreads),
                        _ptr(C), _ptr(D))
    return C, D


def repack(qweight: np.ndarray, K: int, N: int) -> np.ndarray:
    """Tile-order blob (uint32, K*N/8 words) built from the written layout definition."""
    _check_shapes(K, N)
    if N % 16:
        raise ValueError("oracle.repack: N must be a multiple of 16")
    qw = np.ascontiguousarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    out = np.empty(K * N // 8, dtype=np.uint32)
    _load().oracle_repack(_ptr(qw), K, N, _ptr(out))
    return out


def unrepack(blob: np.ndarray, K: int, N: int) -> np.ndarray:
    """Inverse of ``repack``: GPTQ words uint32 [K/8, N]."""
    _check_shapes(K, N)
    b = np.ascontiguousarray(blob, dtype=np.uint32).reshape(-1)
    if b.size != K * N // 8:
        raise ValueError("oracle.unrepack: blob size mismatch")
    out = np.empty((K // 8, N), dtype=np.uint32)
    _load().oracle_unrepack(_ptr(b), K, N, _ptr(out))
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# ---------------------------------------------------------------------------
# bf16 helpers (exact reading; RNE only for values already exact in fp32)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_exact_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bf16 of values that are exactly representable in fp32.

    Raises if a value is not fp32-exact, so that no double rounding can hide here.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("f32_exact_to_bf16_bits: input is not exactly representable in fp32")
    u = f.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rem = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    up = (rem > half) | ((rem == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    out = keep + up.astype(np.uint64)
    return out.astype(np.uint16)


# ---------------------------------------------------------------------------
# Exact rational reference (tiny shapes only)
# ---------------------------------------------------------------------------

def _bf16_fraction(bits: int) -> Fraction:
    """Exact rational value of a finite bf16 bit pattern, from its fields."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite bf16 in exact reference")
    if exp == 0:
        val = Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    else:
        val = (1 + Fraction(man, 1 << 7)) * (Fraction(2) ** (exp - 127))
    return sign * val


def exact_gemm(A_bits, qweight, scales_bits, M: int, N: int, K: int):
    """C[m][n] = sum_k a * (q - 8) * s with exact rationals, and D = sum |a*w|.

    Pure-Python loops; the code of (k, n) is read with integer operations from
    word (k // 8, n), nibble k % 8, low nibble first.
    """
    A_bits = np.asarray(A_bits, dtype=np.uint16).reshape(-1, K)
    qw = np.asarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    sc = np.asarray(scales_bits, dtype=np.uint16).reshape(K // GROUP, N)
    a = [[_bf16_fraction(int(A_bits[m, k])) for k in range(K)] for m in range(M)]
    C = [[Fraction(0)] * N for _ in range(M)]
    D = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            word = int(qw[k // 8, n])
            q = (word >> (4 * (k % 8))) & 0xF
            w = (q - 8) * _bf16_fraction(int(sc[k // GROUP, n]))
            for m in range(M):
                p = a[m][k] * w
                C[m][n] += p
                D[m][n] += abs(p)
    return C, D


# ---------------------------------------------------------------------------
# Acceptance metric
# ---------------------------------------------------------------------------

def silu(x) -> np.ndarray:
    """silu(x) = x / (1 + exp(-x)) in fp64.

    For x < 0 the equal form x * e^x / (1 + e^x) is used, so exp never
    overflows for finite x (silu(-1e6) is -0, not NaN).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = x[pos] / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = x[~pos] * e / (1.0 + e)
    return out


def silu_derivative(x) -> np.ndarray:
    """d/dx silu(x) = s(x) * (1 + x * (1 - s(x))) with s the logistic function."""
    x = np.asarray(x, dtype=np.float64)
    s = np.empty_like(x)
    pos = x >= 0
    s[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    s[~pos] = e / (1.0 + e)
    return s * (1.0 + x * (1.0 - s))


def gemm_silu_mul(A: np.ndarray, qweight: np.ndarray, scales: np.ndarray, M: int, N: int, K: int,
                  js=None, nthreads: int = 0):
    """fp64 reference of the gate/up matmul with its activation:

        H[m, j] = silu(C[m, j]) * C[m, j + N/2],   C = A . dequant(W)  (fp64, as ``gemm``)

    Reading taken (the pages name gate, up and down linears per MLP but not
    the activation or the column order): the first N/2 columns of the fused
    weight are the gate linear, the last N/2 the up linear, and the gating
    is SiLU.  ``js`` selects columns j of H (all N/2 if None).

    Returns (H, E), float64 [M, len(js)].  E = |silu'(g)| |u| D_g + |silu(g)| D_u
    is the first-order change of H when the gate and up sums move by at most
    their own sum |a*w| (D_g, D_u): the GEMM's normalized error bound
    carried through the activation.
    """
    j, cols = _gate_up_columns(N, js, "gemm_silu_mul")
    C, D = gemm(A, qweight, scales, M, N, K, cols=cols, nthreads=nthreads)
    return _silu_mul(C, D, j.size)


def _gate_up_columns(N: int, js, who: str):
    if N % 32:
        raise ValueError(f"oracle.{who}: N must be a multiple of 32")
    half = N // 2
    j = np.arange(half, dtype=np.int64) if js is None else np.asarray(js, dtype=np.int64)
    if j.size and (j.min() < 0 or j.max() >= half):
        raise ValueError(f"oracle.{who}: column index out of range")
    return j, np.concatenate([j, j + half])


def _silu_mul(C, D, nj: int):
    """(H, E) from the gate sums C[:, :nj] and up sums C[:, nj:] and their D."""
    g, u = C[:, :nj], C[:, nj:]
    dg, du = D[:, :nj], D[:, nj:]
    H = silu(g) * u
    E = np.abs(silu_derivative(g)) * np.abs(u) * dg + np.abs(silu(g)) * du
    return H, E


def row_argmax(C: np.ndarray) -> np.ndarray:
    """Column of each row's largest value, the lowest one among equal values
    (numpy's argmax returns the first occurrence; -0 and +0 compare equal)."""
    return np.argmax(np.asarray(C, dtype=np.float64), axis=1)


def normalized_error(C_test: np.ndarray, C_ref: np.ndarray, D_ref: np.ndarray) -> np.ndarray:
    """Per-output error |C_test - C_ref| / D_ref.

    Where D_ref == 0 every term a*w is zero, so the exact result is zero and
    C_test must be +-0: the error there is 0 if it is, +inf otherwise.
    """
    C_test = np.asarray(C_test, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    D_ref = np.asarray(D_ref, dtype=np.float64)
    num = np.abs(C_test - C_ref)
    out = np.empty_like(num)
    nz = D_ref > 0
    out[nz] = num[nz] / D_ref[nz]
    out[~nz] = np.where(C_test[~nz] == 0.0, 0.0, np.inf)
    return out


# ---------------------------------------------------------------------------
# NVFP4 weight-only variant (nvfp4.c)
# ---------------------------------------------------------------------------

NVFP4_BLOCK = 16


def _check_nvfp4(K: int, N: int, multiple: int = GROUP):
    if K % multiple or K <= 0 or N <= 0:
        raise ValueError(f"oracle: K must be a positive multiple of {multiple}, N positive")


def e2m1_to_f64(codes) -> np.ndarray:
    """Values of 4-bit E2M1 codes (sign, 2-bit exponent with bias 1, 1-bit mantissa)."""
    c = np.asarray(codes, dtype=np.int64)
    f = _load().oracle_e2m1_to_f64
    return np.array([f(int(x) & 0xF) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_to_f64(bytes_) -> np.ndarray:
    """Values of FP8 E4M3 bytes (bias 7, subnormals, S.1111.111 = NaN, no infinities)."""
    b = np.asarray(bytes_, dtype=np.int64)
    f = _load().oracle_e4m3_to_f64
    return np.array([f(int(x) & 0xFF) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


def nvfp4_unpack(packed: np.ndarray, K: int, N: int) -> np.ndarray:
    """Codes [K, N] in [0, 15] from packed uint8 [N, K/2] (low nibble = even k)."""
    _check_nvfp4(K, N, 2)
    pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(N, K // 2)
    out = np.empty((K, N), dtype=np.uint8)
    _load().oracle_nvfp4_unpack(_ptr(pk), K, N, _ptr(out))
    return out


def nvfp4_dequant(packed: np.ndarray, scales: np.ndarray, K: int, N: int) -> np.ndarray:
    """W[k, n] = e2m1(code) * e4m3(scale[n, k // 16]) in fp64, without the per-tensor factor."""
    _check_nvfp4(K, N, NVFP4_BLOCK)
    pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(N, K // 2)
    sc = np.ascontiguousarray(scales, dtype=np.uint8).reshape(N, K // NVFP4_BLOCK)
    out = np.empty((K, N), dtype=np.float64)
    _load().oracle_nvfp4_dequant(_ptr(pk), _ptr(sc), K, N, _ptr(out))
    return out


def nvfp4_gemm(A: np.ndarray, packed: np.ndarray, scales: np.ndarray, alpha: float, M: int, N: int,
               K: int, cols=None, nthreads: int = 0):
    """fp64 reference C[M, ncols] = alpha * A . W[:, cols] and D = |alpha| * sum |a*w|.

    ``A`` is bf16 bits [M, K]; ``alpha`` is used at its exact value (pass an
    fp32-representable number to match a caller that holds it in fp32).
    """
    _check_nvfp4(K, N, NVFP4_BLOCK)
    if not 1 <= M <= 16:
        raise ValueError("oracle.nvfp4_gemm: 1 <= M <= 16")
    a = np.ascontiguousarray(np.ascontiguousarray(A, dtype=np.uint16).reshape(-1, K)[:M])
    pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(N, K // 2)
    sc = np.ascontiguousarray(scales, dtype=np.uint8).reshape(N, K // NVFP4_BLOCK)
    if cols is None:
        ncols, cptr = N, None
    else:
        c = np.ascontiguousarray(cols, dtype=np.int32)
        if c.size and (c.min() < 0 or c.max() >= N):
            raise ValueError("oracle.nvfp4_gemm: column index out of range")
        ncols, cptr = int(c.size), _ptr(c)
    C = np.empty((M, ncols), dtype=np.float64)
    D = np.empty((M, ncols), dtype=np.float64)
    _load().oracle_nvfp4_gemm(_ptr(a), _ptr(pk), _ptr(sc), float(alpha), M, N, K, cptr, ncols,
                              int(nthreads), _ptr(C), _ptr(D))
    return C, D


def nvfp4_gemm_silu_mul(A: np.ndarray, packed: np.ndarray, scales: np.ndarray, alpha: float, M: int,
                        N: int, K: int, js=None, nthreads: int = 0):
    """fp64 reference of the gate/up activation on NVFP4 weights:

        H[m, j] = silu(C[m, j]) * C[m, j + N/2],   C = alpha * A . dequant(W)  (as ``nvfp4_gemm``)

    The same reading of the gate/up layout and the same first-order bound E
    as ``gemm_silu_mul``, with D = |alpha| sum |a*w|.  Returns (H, E).
    """
    j, cols = _gate_up_columns(N, js, "nvfp4_gemm_silu_mul")
    C, D = nvfp4_gemm(A, packed, scales, alpha, M, N, K, cols=cols, nthreads=nthreads)
    return _silu_mul(C, D, j.size)


def nvfp4_repack(packed: np.ndarray, K: int, N: int) -> np.ndarray:
    """Tile-order blob (uint8, K*N/2 bytes) built from the written layout definition."""
    _check_nvfp4(K, N)
    if N % 16:
        raise ValueError("oracle.nvfp4_repack: N must be a multiple of 16")
    pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(N, K // 2)
    out = np.empty(K * N // 2, dtype=np.uint8)
    _load().oracle_nvfp4_repack(_ptr(pk), K, N, _ptr(out))
    return out


def nvfp4_unrepack(blob: np.ndarray, K: int, N: int) -> np.ndarray:
    """Inverse of ``nvfp4_repack``: packed uint8 [N, K/2]."""
    _check_nvfp4(K, N)
    if N % 16:
        raise ValueError("oracle.nvfp4_unrepack: N must be a multiple of 16")
    b = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    out = np.empty((N, K // 2), dtype=np.uint8)
    _load().oracle_nvfp4_unrepack(_ptr(b), K, N, _ptr(out))
    return out


def nvfp4_repack_scales(scales: np.ndarray, K: int, N: int) -> np.ndarray:
    """Scales [N, K/16] -> [tile][superblock][16 columns][8 blocks] (uint8)."""
    _check_nvfp4(K, N)
    if N % 16:
        raise ValueError("oracle.nvfp4_repack_scales: N must be a multiple of 16")
    sc = np.ascontiguousarray(scales, dtype=np.uint8).reshape(N, K // NVFP4_BLOCK)
    out = np.empty(K * N // NVFP4_BLOCK, dtype=np.uint8)
    _load().oracle_nvfp4_repack_scales(_ptr(sc), K, N, _ptr(out))
    return out


def _e2m1_fraction(code: int) -> Fraction:
    sign = -1 if code & 8 else 1
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2 + m, 2) * Fraction(2) ** (e - 1)
    return sign * mag


def _e4m3_fraction(byte: int) -> Fraction:
    sign = -1 if byte & 0x80 else 1
    e, m = (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        raise ValueError("E4M3 NaN has no rational value")
    mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return sign * mag


def nvfp4_exact_gemm(A_bits, packed, scale_bytes, alpha: Fraction, M: int, N: int, K: int):
    """Exact rational C for tiny shapes (Python integers and Fractions only).

    Each element and scale is decoded from its bit fields by the format
    definition, independently of nvfp4.c.
    """
    A_bits = np.asarray(A_bits, dtype=np.uint16).reshape(-1, K)
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)
    scale_bytes = np.asarray(scale_bytes, dtype=np.uint8).reshape(N, K // NVFP4_BLOCK)
    out = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            byte = int(packed[n, k // 2])
            code = byte & 0xF if k % 2 == 0 else byte >> 4
            w = alpha * _e2m1_fraction(code) * _e4m3_fraction(int(scale_bytes[n, k // NVFP4_BLOCK]))
            if w == 0:
                continue
            for m in range(M):
                out[m][n] += _bf16_fraction(int(A_bits[m, k])) * w
    return out
