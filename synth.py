"""Seeded synthetic inputs for the W4A16 matmul (shared by the oracle tests and the HIP path).

This module draws random inputs and nothing else: it holds none of the
matmul's arithmetic (no unpacking, dequantization, repacking or products).

Distributions follow the workloads of the W4A16 decode/verify matmul on a dense
27B hybrid model (geometry from the page "Qwen3.8 27B - NVFP4 for veloGB10",
section "Specifications": hidden 5120, 24 Q / 4 KV heads of head_dim 256,
64 layers, vocabulary 248,320):

* codes: uniform on [0, 15], packed 8 per uint32 along K, low nibble first.
  A uniform 32-bit word has 8 independent nibbles each uniform on [0, 15], so
  the packed words are drawn directly as uniform uint32.
* scales: bf16(|N(0,1)| * 0.01), one per (K group of 128, column), [K/128, N].
* activations A: bf16(N(0,1)), [M, K]; for the MLP down projection
  bf16(SiLU(x) * y) with x, y ~ N(0,1) i.i.d., SiLU(x) = x / (1 + exp(-x)),
  computed in fp64, rounded to fp32, then to bf16.
* every float -> bf16 conversion is round-to-nearest-even on the fp32 bits.

Draw order from ``numpy.random.default_rng(seed)``: words, then scales, then A
(16 rows; an M-row call uses the first M rows).

NVFP4 weight-only variant (same shapes, seeds offset by 10):

* codes: uniform bytes, i.e. two independent uniform 4-bit E2M1 codes per
  byte (all 16 codes, -0 included), packed uint8 [N, K/2];
* block scales: E4M3 bytes with sign 0, exponent field uniform on [4, 10] and
  mantissa uniform on [0, 7] (values 2^-3 .. 1.875 * 2^3: finite and
  positive, as a block maximum over 6 is after a per-tensor factor), uint8
  [N, K/16];
* per-tensor factor: fp32(0.0037);
* A as above; draw order codes, scales, A.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 128
M_MAX = 16


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    K: int
    N: int
    Ms: tuple
    seed: int
    act: str = "normal"       # "normal" or "silu_mul"
    desc: str = ""

    @property
    def groups(self) -> int:
        return self.K // GROUP


# The workloads, with the shapes of a dense 27B hybrid model's linear layers.
WORKLOADS = {
    "tiny": Workload("tiny", 512, 1024, (1,), 0, desc="Tiny W4A16: M=1, K=512, N=1024"),
    "qkv": Workload("qkv", 5120, 8192, (1,), 1,
                    desc="QKV-shaped decode: K=5120, N=8192 (24 Q heads + 2x4 KV heads, head_dim 256)"),
    "gate_up": Workload("gate_up", 5120, 34816, (1, 2, 4, 8, 9, 16), 2,
                        desc="Fused gate/up MLP: K=5120, N=34816 (2x17408)"),
    "down": Workload("down", 17408, 5120, (1, 4, 8, 16), 3, act="silu_mul",
                     desc="Down projection: K=17408, N=5120, A = SiLU(x)*y"),
    "attn_out": Workload("attn_out", 6144, 5120, (1, 2, 4, 8, 16), 5,
                         desc="Attention output projection: K=6144 (24 heads x 256), N=5120"),
    "lm_head": Workload("lm_head", 5120, 248320, (1, 8, 16), 4,
                        desc="Output head: K=5120, N=248320"),
}

# One decode step's linear shapes for the full-stack sweep: every one of the 64
# layers gets an attention-in (5120 -> 8192), attention-out (6144 -> 5120),
# gate/up (5120 -> 34816) and down (17408 -> 5120) projection; lm_head runs once.
STACK_LAYER_SHAPES = ((5120, 8192), (6144, 5120), (5120, 34816), (17408, 5120))
STACK_LAYERS = 64
LM_HEAD_SHAPE = (5120, 248320)


def gen_weights(K: int, N: int, rng: np.random.Generator):
    """(qweight uint32 [K/8, N], scales bf16 bits uint16 [K/128, N])."""
    if K % GROUP or N <= 0:
        raise ValueError("K must be a multiple of 128")
    qweight = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint32)
    s = np.abs(rng.standard_normal((K // GROUP, N))) * 0.01
    scales = _f32_to_bf16_bits(s)
    return qweight, scales


def gen_activations(M: int, K: int, rng: np.random.Generator, act: str = "normal"):
    """A as bf16 bits uint16 [M, K]."""
    if act == "normal":
        a = rng.standard_normal((M, K))
    elif act == "silu_mul":
        x = rng.standard_normal((M, K))
        y = rng.standard_normal((M, K))
        a = x / (1.0 + np.exp(-x)) * y
    else:
        raise ValueError(f"unknown activation distribution {act!r}")
    return _f32_to_bf16_bits(a)


def gen_problem(K: int, N: int, seed: int, act: str = "normal", M: int = M_MAX):
    """(A, qweight, scales) for one seeded problem, drawn in the documented order."""
    rng = np.random.default_rng(seed)
    qweight, scales = gen_weights(K, N, rng)
    A = gen_activations(M, K, rng, act)
    return A, qweight, scales


def gen_workload(name: str, M: int = M_MAX):
    w = WORKLOADS[name]
    return gen_problem(w.K, w.N, w.seed, w.act, M)


NVFP4_BLOCK = 16
NVFP4_SEED_OFFSET = 10
NVFP4_ALPHA = float(np.float32(0.0037))


def gen_nvfp4_weights(K: int, N: int, rng: np.random.Generator):
    """(packed codes uint8 [N, K/2], E4M3 scale bytes uint8 [N, K/16])."""
    if K % GROUP or N <= 0:
        raise ValueError("K must be a multiple of 128")
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    e = rng.integers(4, 11, size=(N, K // NVFP4_BLOCK), dtype=np.uint8)
    m = rng.integers(0, 8, size=(N, K // NVFP4_BLOCK), dtype=np.uint8)
    return packed, ((e << 3) | m).astype(np.uint8)


def gen_nvfp4_problem(K: int, N: int, seed: int, act: str = "normal", M: int = M_MAX):
    """(A, packed, scale bytes) for one seeded NVFP4 problem, drawn in the documented order."""
    rng = np.random.default_rng(seed)
    packed, scales = gen_nvfp4_weights(K, N, rng)
    A = gen_activations(M, K, rng, act)
    return A, packed, scales


def gen_nvfp4_workload(name: str, M: int = M_MAX):
    w = WORKLOADS[name]
    return gen_nvfp4_problem(w.K, w.N, w.seed + NVFP4_SEED_OFFSET, w.act, M)


def algorithmic_bytes_nvfp4(M: int, N: int, K: int) -> int:
    """Bytes of one NVFP4 call: 4-bit codes, one E4M3 byte per 16 weights, bf16 A, bf16 C."""
    return K * N // 2 + (K // NVFP4_BLOCK) * N + M * K * 2 + M * N * 2


def algorithmic_bytes_silu_mul(M: int, N: int, K: int) -> int:
    """Bytes of the gate/up call with its activation: codes, scales, A, and H[M, N/2] written."""
    return K * N // 2 + (K // GROUP) * N * 2 + M * K * 2 + M * (N // 2) * 2


def algorithmic_bytes_argmax(M: int, N: int, K: int) -> int:
    """Bytes of the output projection with its row argmax: codes, scales, A, and M (index, value) pairs."""
    return K * N // 2 + (K // GROUP) * N * 2 + M * K * 2 + M * 8


def algorithmic_bytes_f32(M: int, N: int, K: int) -> int:
    """Bytes of a K shard's call: codes, scales, A, and fp32 partial sums C[M, N] written."""
    return K * N // 2 + (K // GROUP) * N * 2 + M * K * 2 + M * N * 4


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """Bytes one call must move at least: int4 codes, bf16 scales, bf16 A, bf16 C."""
    return K * N // 2 + (K // GROUP) * N * 2 + M * K * 2 + M * N * 2
