"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bars (from the acceptance rule for this matmul):
  * repack blob, unpacked codes and fp32 dequantized weights: bit-exact;
  * C: max over outputs of |C_gpu - C_ref| / sum_k |a_k w_k| <= 2e-3, with
    C_ref and the normalizer from the fp64 oracle on the same seeded inputs;
  * special inputs whose exact result is representable: bitwise equal to the
    round-to-nearest-even bf16 of the exact value;
  * repeated calls and row prefixes: bitwise equal.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_gptq_amd as w4

pytestmark = pytest.mark.gpu
TOL = 2e-3
DEV = "cuda:0"


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(qweight, scales, A=None):
    """Device copies: GPTQ words, the checkpoint's bf16 scales [K/128, N], bf16 A."""
    q = torch.from_numpy(qweight.view(np.int32)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).to(DEV).view(torch.bfloat16)
    a = None if A is None else torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).to(DEV).view(torch.bfloat16)
    return q, s, a


def c_bits(C):
    return C.view(torch.int16).cpu().numpy().view(np.uint16)


def run_gemm(a, blob, s, N, M, plan=None, ws=None):
    out = w4.gemm(a[:M].contiguous(), blob, s, N, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    return out


def max_err(C, Cref, Dref):
    e = oracle.normalized_error(oracle.bf16_bits_to_f64(c_bits(C)), Cref, Dref)
    return float(e.max())


# ------------------------------------------------------------- plans to force
# every (path, tiles, kwaves, A source, ring depth) combination a build might
# hold; plan_ok keeps the ones the library has kernels for (depth 0 = its default)
ALL_PLANS = []
for path in (w4.PATH_GEMV, w4.PATH_MFMA):
    for t in (1, 2, 4, 8):
        for kw in (1, 2, 4, 5, 8, 10, 16):
            for asrc in ((w4.ASRC_LDS,) if path == w4.PATH_GEMV
                         else (w4.ASRC_LDS, w4.ASRC_GLOBAL, w4.ASRC_RING, w4.ASRC_SPLITN)):
                for depth in (0, 2, 3, 4, 5, 8, 10, 17):
                    ALL_PLANS.append(w4.make_plan(path, t, kw, 1, asrc, depth))


def plans_for(M, N, K):
    """Every single-split plan the library has a kernel for at (M, N, K)."""
    return [p for p in ALL_PLANS if w4.plan_ok(M, N, K, p)]


# ------------------------------------------------------------- bit-exact weights

@pytest.mark.parametrize("K,N,seed", [(128, 16, 1), (512, 1024, 0), (1152, 592, 2), (5120, 8192, 1)])
def test_repack_unpack_dequant_bit_exact(K, N, seed):
    note(f"[repack/unpack/dequant] K={K} N={N} seed={seed}")
    _, qw, sc = synth.gen_problem(K, N, seed, M=1)
    q, s, _ = to_dev(qw, sc)
    blob = w4.repack_weights(q, K, N)
    codes = w4.unpack_debug(blob, K, N)
    W = w4.dequant_debug(blob, s, K, N)
    torch.cuda.synchronize()
    ref_blob = oracle.repack(qw, K, N)
    assert np.array_equal(blob.cpu().numpy().view(np.uint32), ref_blob)
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack(qw, K, N))
    Wd = W.cpu().numpy().astype(np.float64)
    assert np.array_equal(Wd, oracle.dequant(qw, sc, K, N))


def test_dequant_subnormal_and_extreme_scales():
    K, N = 256, 32
    _, qw, _ = synth.gen_problem(K, N, 9, M=1)
    sc = np.zeros((K // 128, N), dtype=np.uint16)
    sc[0, :] = np.arange(1, N + 1, dtype=np.uint16)            # subnormal bf16
    # large scales, just below the point where 8 * s leaves the fp32 range
    # (above it the fp32 export correctly overflows where fp64 does not)
    sc[1, :] = 0x7D00 + np.arange(N, dtype=np.uint16)          # about 2^123 .. 2^124
    q, s, _ = to_dev(qw, sc)
    blob = w4.repack_weights(q, K, N)
    W = w4.dequant_debug(blob, s, K, N)
    torch.cuda.synchronize()
    assert np.array_equal(W.cpu().numpy().astype(np.float64), oracle.dequant(qw, sc, K, N))


# ------------------------------------------------------------- GEMM, all plans

SMALL_SHAPES = [(512, 1024, 0), (1152, 592, 5), (384, 48, 6), (128, 16, 7), (2048, 272, 8)]


@pytest.mark.parametrize("K,N,seed", SMALL_SHAPES)
def test_gemm_parity_every_plan_every_m(K, N, seed):
    A, qw, sc = synth.gen_problem(K, N, seed)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Cref16, Dref16 = oracle.gemm(A, qw, sc, 16, N, K)
    worst = 0.0
    for M in range(1, 17):
        cases = [None] + plans_for(M, N, K)
        note(f"[gemm] K={K} N={N} M={M}: {len(cases)} plans")
        for p in cases:
            C = run_gemm(a, blob, s, N, M, plan=p)
            e = max_err(C, Cref16[:M], Dref16[:M])
            worst = max(worst, e)
            assert e <= TOL, (M, p, e)
    note(f"  worst normalized error {worst:.3e}")


def test_ring_tail_every_remainder():
    # the ring driver's three ways to end: whole rounds, the exact tail with
    # rt = ng mod D refills left (one compiled tail per rt, depths 2..4),
    # and fewer groups than slots; K = 128 * G with G = 1..11 groups and one
    # wavefront along K (ng = G), so every rt and every ng < D occurs for
    # each depth; GEMV, staged, global and ring A; bitwise repeatable
    N = 64
    for G in range(1, 12):
        K = 128 * G
        A, qw, sc = synth.gen_problem(K, N, 60 + G)
        q, s, a = to_dev(qw, sc, A)
        blob = w4.repack_weights(q, K, N)
        Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K)
        ran = 0
        for M in (1, 3, 8, 16):
            for path in (w4.PATH_GEMV, w4.PATH_MFMA):
                for asrc in ((w4.ASRC_LDS,) if path == w4.PATH_GEMV else (w4.ASRC_LDS, w4.ASRC_GLOBAL, w4.ASRC_RING)):
                    for t, kw in ((1, 1), (2, 1), (1, 4), (2, 4), (1, 8)):
                        for d in (2, 3, 4, 5, 8, 10):
                            p = w4.make_plan(path, t, kw, 1, asrc, d)
                            if not w4.plan_ok(M, N, K, p):
                                continue
                            C1 = run_gemm(a, blob, s, N, M, plan=p)
                            C2 = run_gemm(a, blob, s, N, M, plan=p)
                            e = max_err(C1, Cref[:M], Dref[:M])
                            assert e <= TOL, (G, M, p, e)
                            assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), (G, M, p)
                            ran += 1
        note(f"[ring tail] G={G}: {ran} plans")
        assert ran > 0


@pytest.mark.parametrize("K,N,seed", [(5120, 96, 9), (17408, 48, 10)])
def test_gemm_parity_every_plan_long_k(K, N, seed):
    # K = 5120 (40 groups) and 17408 (136 groups): wavefront group counts that
    # are multiples of the ring depth (every refill real, last round loads
    # nothing) and ones that are not (clamped refills), for every depth
    A, qw, sc = synth.gen_problem(K, N, seed)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Cref16, Dref16 = oracle.gemm(A, qw, sc, 16, N, K)
    for M in (1, 2, 4, 5, 16):
        cases = [None] + plans_for(M, N, K)
        note(f"[gemm long K] K={K} N={N} M={M}: {len(cases)} plans")
        for p in cases:
            C = run_gemm(a, blob, s, N, M, plan=p)
            e = max_err(C, Cref16[:M], Dref16[:M])
            assert e <= TOL, (M, p, e)


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_gemm_split_k_parity_and_reuse(splits):
    K, N = 1280, 528
    A, qw, sc = synth.gen_problem(K, N, 21)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K)
    for M in (1, 3, 4, 8, 16):
        for path, asrc in ((w4.PATH_GEMV, 0), (w4.PATH_MFMA, 0), (w4.PATH_MFMA, 1), (w4.PATH_MFMA, 2), (w4.PATH_MFMA, 3)):
            if path == w4.PATH_GEMV and M > 4:
                continue
            for t, kw in ((1, 4), (2, 8)):
                p = w4.make_plan(path, t, kw, splits, asrc)
                if not w4.plan_ok(M, N, K, p):
                    p = w4.make_plan(path, t * 2, 4, splits, asrc)   # ring A: (2, 4) / (4, 4) shapes
                nbytes = w4.workspace_bytes(M, N, K, p)
                assert nbytes > 0
                ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
                note(f"[split-k] M={M} plan={p}")
                C1 = run_gemm(a, blob, s, N, M, plan=p, ws=ws)
                C2 = run_gemm(a, blob, s, N, M, plan=p, ws=ws)   # counters were reset
                assert max_err(C1, Cref[:M], Dref[:M]) <= TOL
                assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
                assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("K,N,seed", [(1280, 528, 23), (17408, 48, 24), (2048, 1040, 25)])
def test_gemm_remainder_split_parity(K, N, seed):
    # the leading strips whole, the rest split along K: every path and A
    # source, split counts 2 and 4, nothing / one / half / all but one /
    # every strip whole; repeated calls are bitwise equal and leave the
    # counters zero
    A, qw, sc = synth.gen_problem(K, N, seed)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K)
    shapes = [(w4.PATH_GEMV, 1, 8, 2, w4.ASRC_LDS), (w4.PATH_GEMV, 2, 4, 3, w4.ASRC_LDS),
              (w4.PATH_MFMA, 1, 8, 2, w4.ASRC_RING), (w4.PATH_MFMA, 2, 4, 4, w4.ASRC_LDS),
              (w4.PATH_MFMA, 2, 4, 4, w4.ASRC_GLOBAL), (w4.PATH_MFMA, 2, 4, 2, w4.ASRC_RING),
              (w4.PATH_MFMA, 1, 4, 4, w4.ASRC_SPLITN), (w4.PATH_MFMA, 2, 4, 3, w4.ASRC_SPLITN)]
    ws = torch.zeros(65536 + 4 * 16 * N * 4, dtype=torch.uint8, device=DEV)
    ran = 0
    for M in (1, 3, 4, 8, 13, 16):
        for (path, t, kw, d, asrc) in shapes:
            nstrips = -(-(N // 16) // (t * (kw if asrc == w4.ASRC_SPLITN else 1)))
            for S in (2, 4):
                for whole in sorted({0, 1, nstrips // 2, nstrips - 1, nstrips}):
                    p = w4.make_plan(path, t, kw, S, asrc, d, whole)
                    if not w4.plan_ok(M, N, K, p):
                        continue
                    C1 = run_gemm(a, blob, s, N, M, plan=p, ws=ws)
                    C2 = run_gemm(a, blob, s, N, M, plan=p, ws=ws)
                    e = max_err(C1, Cref[:M], Dref[:M])
                    assert e <= TOL, (M, p, e)
                    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), (M, p)
                    ran += 1
    note(f"[remainder split] K={K} N={N}: {ran} plans")
    assert ran > 50
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_split_k_workspace_shared_across_shapes():
    # one zero-filled workspace serves split calls of different M, N, splits
    # and tiles in stream order: each call's partials stay clear of the
    # counter region every call leaves at zero
    cases = []
    for (K, N, seed) in ((17408, 48, 10), (1280, 528, 21), (2048, 272, 8)):
        A, qw, sc = synth.gen_problem(K, N, seed)
        q, s, a = to_dev(qw, sc, A)
        blob = w4.repack_weights(q, K, N)
        Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K)
        cases.append((K, N, a, blob, s, Cref, Dref))
    plans = [w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_LDS), w4.make_plan(w4.PATH_MFMA, 4, 4, 2, w4.ASRC_GLOBAL),
             w4.make_plan(w4.PATH_GEMV, 1, 4, 8), w4.make_plan(w4.PATH_MFMA, 1, 8, 2, w4.ASRC_GLOBAL),
             w4.make_plan(w4.PATH_MFMA, 4, 4, 2, w4.ASRC_RING), w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_SPLITN),
             w4.make_plan(w4.PATH_GEMV, 1, 8, 4, w4.ASRC_LDS, 2, 2), w4.make_plan(w4.PATH_MFMA, 1, 8, 2, w4.ASRC_RING, 2, 1)]
    need = max(w4.workspace_bytes(16, N, K, p) for (K, N, *_) in cases for p in plans)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for rnd in range(2):
        for (K, N, a, blob, s, Cref, Dref) in cases:
            for M in (4, 5, 2, 16, 1):
                for p in [None] + plans:
                    if p is not None and (not w4.plan_ok(M, N, K, p)):
                        continue
                    C = run_gemm(a, blob, s, N, M, plan=p, ws=ws)
                    e = max_err(C, Cref[:M], Dref[:M])
                    assert e <= TOL, (rnd, K, N, M, p, e)
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


# ------------------------------------------------------------- exact special inputs

def _pow2_bf16(e):
    return ((127 + e) & 0xFF) << 7


@pytest.mark.parametrize("word,colsum", [(0x76543210, -36), (0xFEDCBA98, 28), (0xFFFFFFFF, 56),
                                          (0x00000000, -64), (0x88888888, 0)])
def test_gemm_exact_ones(word, colsum):
    # A = ones, s = 2^-3: C = 2^-3 * (K/8) * colsum exactly (an integer < 2^24 times 2^-3)
    K, N = 2048, 64
    A = np.full((16, K), 0x3F80, dtype=np.uint16)
    qw = np.full((K // 8, N), word, dtype=np.uint32)
    sc = np.full((K // 128, N), _pow2_bf16(-3), dtype=np.uint16)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    exact = colsum * (K // 8) * 2.0 ** -3
    expect = int(oracle.f32_exact_to_bf16_bits(np.array([exact]))[0])
    for M in (1, 2, 4, 8, 16):
        for p in [None] + plans_for(M, N, K):
            C = run_gemm(a, blob, s, N, M, plan=p)
            assert np.all(c_bits(C) == expect), (M, p)


def test_gemm_exact_one_hot_rows_and_groups():
    # q-8 = k % 8 everywhere; s[g, n] = 2^(g - n % 3); row m of A is one-hot at k_m
    K, N = 1024, 48
    qw = np.full((K // 8, N), 0xFEDCBA98, dtype=np.uint32)
    sc = np.array([[_pow2_bf16(g - n % 3) for n in range(N)] for g in range(K // 128)], dtype=np.uint16)
    ks = [0, 5, 127, 128, 129, 255, 300, 511, 512, 640, 777, 895, 896, 1000, 1022, 1023]
    A = np.zeros((16, K), dtype=np.uint16)
    for m, k in enumerate(ks):
        A[m, k] = 0x3F80
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    expect = np.array([[(k % 8) * 2.0 ** (k // 128 - n % 3) for n in range(N)] for k in ks])
    ebits = oracle.f32_exact_to_bf16_bits(expect)
    for M in (1, 4, 9, 16):
        for p in [None] + plans_for(M, N, K):
            C = run_gemm(a, blob, s, N, M, plan=p)
            assert np.array_equal(c_bits(C), ebits[:M]), (M, p)


def test_gemm_zero_weights_give_signed_zero_free_exact_zero():
    K, N = 512, 32
    A, _, sc = synth.gen_problem(K, N, 3)
    qw = np.full((K // 8, N), 0x88888888, dtype=np.uint32)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    for M in (1, 4, 16):
        C = run_gemm(a, blob, s, N, M)
        assert np.all(oracle.bf16_bits_to_f64(c_bits(C)) == 0.0)


# ------------------------------------------------------------- determinism

def test_determinism_and_row_prefix():
    K, N = 5120, 2048
    A, qw, sc = synth.gen_problem(K, N, 31)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    for p in plans_for(16, N, K):
        C16 = run_gemm(a, blob, s, N, 16, plan=p)
        C16b = run_gemm(a, blob, s, N, 16, plan=p)
        assert torch.equal(C16.view(torch.int16), C16b.view(torch.int16)), p
        for M in (5, 8, 9):
            CM = run_gemm(a, blob, s, N, M, plan=p)
            assert torch.equal(CM.view(torch.int16), C16[:M].view(torch.int16)), (M, p)
    for M in (1, 2, 3, 4):
        C1 = run_gemm(a, blob, s, N, M)
        C2 = run_gemm(a, blob, s, N, M)
        assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


# ------------------------------------------------------------- full workload sizes

# every row count the decode step and the verify batches call each shape
# with, through the automatic plans (the plain kernels the full-stack timing runs)
FULL_MS = {"tiny": (1,), "qkv": (1, 2, 4, 8, 9, 16), "attn_out": (1, 2, 4, 8, 9, 16),
           "gate_up": (1, 2, 4, 8, 9, 16), "down": (1, 2, 3, 4, 5, 8, 9, 12, 13, 16)}


@pytest.mark.parametrize("name", ["tiny", "qkv", "attn_out", "gate_up", "down"])
def test_workload_parity_full(name):
    wl = synth.WORKLOADS[name]
    K, N = wl.K, wl.N
    Ms = FULL_MS[name]
    note(f"[workload] {name} K={K} N={N} Ms={Ms}")
    A, qw, sc = synth.gen_workload(name)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    torch.cuda.synchronize()
    assert np.array_equal(blob.cpu().numpy().view(np.uint32), oracle.repack(qw, K, N))
    Cref, Dref = oracle.gemm(A, qw, sc, max(Ms), N, K)
    for M in Ms:
        C = run_gemm(a, blob, s, N, M)
        e = max_err(C, Cref[:M], Dref[:M])
        note(f"  M={M} plan={w4.get_plan(M, N, K)} max normalized error {e:.3e}")
        assert e <= TOL


def test_workload_parity_lm_head_sampled():
    wl = synth.WORKLOADS["lm_head"]
    K, N = wl.K, wl.N
    A, qw, sc = synth.gen_workload("lm_head")
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    tiles = np.unique(np.concatenate([[0, 1, N // 16 - 1], rng.integers(0, N // 16, 61)]))
    hb = blob.view(torch.int32)
    G = K // 128
    for t in tiles:     # each 16-column tile's chunks are self-contained in the layout
        sub = oracle.repack(np.ascontiguousarray(qw[:, 16 * t:16 * t + 16]), K, 16)
        got = hb[t * G * 256:(t + 1) * G * 256].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, sub), t
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.integers(0, N, 2000)]))
    Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K, cols=cols)
    for M in (1, 8, 16):
        C = run_gemm(a, blob, s, N, M)
        Cs = C[:, torch.from_numpy(cols).to(DEV)]
        e = max_err(Cs, Cref[:M], Dref[:M])
        note(f"  lm_head M={M} plan={w4.get_plan(M, N, K)} max normalized error {e:.3e}")
        assert e <= TOL


# ------------------------------------------------------------- gate/up activation epilogue

def silu_mul_check(H, Href, E, what):
    """|H - Href| <= 2e-3 E (the GEMM bound carried through silu * up) plus one
    bf16 rounding of H (at most 2^-8 |H|)."""
    got = oracle.bf16_bits_to_f64(c_bits(H))
    err = np.abs(got - Href)
    # + 2^-100: the activation runs in fp32, where exp(-g) overflows for
    # g < -88.7 and silu(g) becomes -0; the exact |H| there is below
    # 88 e^-88 |u| < 1e-36 |u|, far under this floor for any |u| < 1e6
    bound = TOL * E * 1.01 + 2.0 ** -8 * np.abs(Href) * (1 + 1e-6) + 2.0 ** -100
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float((err - bound).max()))


EVEN_PLANS = [p for p in ALL_PLANS if p.tiles % 2 == 0]


@pytest.mark.parametrize("K,N,seed", [(512, 1024, 30), (1152, 608, 31), (384, 64, 32), (2048, 288, 33)])
def test_silu_mul_parity_every_even_plan(K, N, seed):
    A, qw, sc = synth.gen_problem(K, N, seed)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Href16, E16 = oracle.gemm_silu_mul(A, qw, sc, 16, N, K)
    for M in (1, 2, 3, 4, 5, 8, 16):
        cases = [None] + [p for p in EVEN_PLANS if w4.plan_ok(M, N, K, p)]
        note(f"[silu-mul] K={K} N={N} M={M}: {len(cases)} plans")
        for p in cases:
            H = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N, plan=p)
            torch.cuda.synchronize()
            silu_mul_check(H, Href16[:M], E16[:M], (M, p))


@pytest.mark.parametrize("splits", [2, 4])
def test_silu_mul_split_k(splits):
    K, N = 1280, 544
    A, qw, sc = synth.gen_problem(K, N, 34)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Href, E = oracle.gemm_silu_mul(A, qw, sc, 16, N, K)
    for M in (1, 4, 9, 16):
        for path, asrc in ((w4.PATH_GEMV, 0), (w4.PATH_MFMA, 0), (w4.PATH_MFMA, 1), (w4.PATH_MFMA, 2), (w4.PATH_MFMA, 3)):
            if path == w4.PATH_GEMV and M > 4:
                continue
            p = w4.make_plan(path, 2, 4, splits, asrc)
            if not w4.plan_ok(M, N, K, p):
                continue
            ws = torch.zeros(w4.workspace_bytes(M, N, K, p), dtype=torch.uint8, device=DEV)
            note(f"[silu-mul split] M={M} plan={p}")
            H1 = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
            H2 = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
            torch.cuda.synchronize()
            silu_mul_check(H1, Href[:M], E[:M], (M, p))
            assert torch.equal(H1.view(torch.int16), H2.view(torch.int16))


def test_epilogue_modes_remainder_split():
    # gate/up activation and fp32 output with the leading strips whole and
    # the rest split along K (the automatic plans of the gate/up width from
    # five rows): split-N, ring and GEMV strips; repeated calls bitwise equal
    K, N = 1280, 1088
    A, qw, sc = synth.gen_problem(K, N, 37)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Href, E = oracle.gemm_silu_mul(A, qw, sc, 16, N, K)
    C16, D16 = oracle.gemm(A, qw, sc, 16, N, K)
    ws = torch.zeros(65536 + 4 * 16 * N * 4, dtype=torch.uint8, device=DEV)
    ran = 0
    for M in (1, 4, 9, 16):
        for (path, t, kw, d, asrc) in ((w4.PATH_MFMA, 2, 4, 3, w4.ASRC_SPLITN), (w4.PATH_MFMA, 2, 4, 2, w4.ASRC_RING),
                                       (w4.PATH_MFMA, 2, 8, 2, w4.ASRC_RING), (w4.PATH_GEMV, 2, 8, 2, w4.ASRC_LDS)):
            nstrips = -(-(N // 16) // (t * (kw if asrc == w4.ASRC_SPLITN else 1)))
            for S in (2, 4):
                for whole in sorted({1, nstrips // 2, nstrips - 1}):
                    p = w4.make_plan(path, t, kw, S, asrc, d, whole)
                    if not w4.plan_ok(M, N, K, p):
                        continue
                    H1 = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
                    H2 = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
                    C = w4.gemm_f32(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
                    torch.cuda.synchronize()
                    silu_mul_check(H1, Href[:M], E[:M], (M, p))
                    assert torch.equal(H1.view(torch.int16), H2.view(torch.int16)), (M, p)
                    e = oracle.normalized_error(C.cpu().numpy().astype(np.float64), C16[:M], D16[:M])
                    assert e.max() <= TOL, (M, p, float(e.max()))
                    ran += 1
    note(f"[epilogue remainder split] {ran} plans")
    assert ran >= 40
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_deep_split_reduction():
    # 16 and 32 pieces per strip: the last workgroup adds the partials in
    # several batches of loads.  Ragged strips (33 tiles; 34 for gate/up):
    # some split-N wavefronts of the last strip hold no tile.  Plain C, the
    # gate/up activation and the fp32 output; repeated calls are bitwise
    # equal and leave the counters zero.
    K = 4096
    ran = 0
    for N in (528, 544):
        A, qw, sc = synth.gen_problem(K, N, 38 + N)
        q, s, a = to_dev(qw, sc, A)
        blob = w4.repack_weights(q, K, N)
        C16, D16 = oracle.gemm(A, qw, sc, 16, N, K)
        Href, E = oracle.gemm_silu_mul(A, qw, sc, 16, N, K) if N == 544 else (None, None)
        shapes = [(w4.PATH_MFMA, 1, 4, 4, w4.ASRC_SPLITN), (w4.PATH_MFMA, 2, 4, 2, w4.ASRC_SPLITN),
                  (w4.PATH_MFMA, 1, 1, 8, w4.ASRC_LDS), (w4.PATH_GEMV, 1, 1, 8, w4.ASRC_LDS),
                  (w4.PATH_MFMA, 1, 4, 4, w4.ASRC_RING)]
        for M in (1, 5, 16):
            for (path, t, kw, d, asrc) in shapes:
                for S in (8, 16, 32):
                    p = w4.make_plan(path, t, kw, S, asrc, d)
                    if not w4.plan_ok(M, N, K, p):
                        continue
                    ws = torch.zeros(w4.workspace_bytes(M, N, K, p), dtype=torch.uint8, device=DEV)
                    note(f"[deep split] N={N} M={M} plan={p}")
                    C1 = run_gemm(a, blob, s, N, M, plan=p, ws=ws)
                    C2 = run_gemm(a, blob, s, N, M, plan=p, ws=ws)
                    e = max_err(C1, C16[:M], D16[:M])
                    assert e <= TOL, (M, p, e)
                    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), (M, p)
                    F = w4.gemm_f32(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
                    torch.cuda.synchronize()
                    ef = oracle.normalized_error(F.cpu().numpy().astype(np.float64), C16[:M], D16[:M])
                    assert ef.max() <= TOL, (M, p, float(ef.max()))
                    if Href is not None and t % 2 == 0:
                        H = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
                        torch.cuda.synchronize()
                        silu_mul_check(H, Href[:M], E[:M], (M, p))
                    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
                    ran += 1
    note(f"[deep split] {ran} plans")
    assert ran >= 40


def test_silu_mul_zero_gate_is_exact_zero_and_odd_tiles_rejected():
    K, N = 512, 256
    A, qw, sc = synth.gen_problem(K, N, 35)
    qw = qw.copy()
    qw[:, : N // 2] = 0x88888888                       # gate weights zero
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    for M in (1, 4, 16):
        H = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N)
        torch.cuda.synchronize()
        assert int((H.view(torch.int16) & 0x7FFF).abs().sum()) == 0
    with pytest.raises(w4.W4A16Error):
        w4.gemm_silu_mul(a[:1].contiguous(), blob, s, N, plan=w4.make_plan(w4.PATH_GEMV, 1, 4))


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 2, 4, 8, 9, 16])
def test_silu_mul_gate_up_workload(M):
    wl = synth.WORKLOADS["gate_up"]
    K, N = wl.K, wl.N
    A, qw, sc = synth.gen_workload("gate_up")
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    js = np.random.default_rng(36).choice(N // 2, size=2048, replace=False)
    Href, E = oracle.gemm_silu_mul(A, qw, sc, M, N, K, js=js)
    H = w4.gemm_silu_mul(a[:M].contiguous(), blob, s, N)
    torch.cuda.synchronize()
    note(f"[silu-mul gate_up] M={M} plan={w4.get_plan(M, N, K).as_dict()}")
    silu_mul_check(H[:, torch.from_numpy(js).to(DEV)], Href, E, M)


# ------------------------------------------------------------- greedy pick (row argmax)

def argmax_check(idx, val, C, D, what):
    """Validity where several columns are within rounding of the maximum: the
    chosen column's exact value is within the GEMM bound of the exact maximum,
    the reported value within the bound of the chosen column's exact value;
    and the exact winner is required wherever the top two are separated by
    more than their bounds."""
    idx = idx.cpu().numpy().astype(np.int64)
    val = val.cpu().numpy().astype(np.float64)
    best = oracle.row_argmax(C)
    rows = np.arange(C.shape[0])
    cg, cb = C[rows, idx], C[rows, best]
    dg, db = D[rows, idx], D[rows, best]
    assert np.all(cg >= cb - TOL * (dg + db)), (what, idx, best)
    assert np.all(np.abs(val - cg) <= TOL * dg + 1e-30), (what, val, cg)
    srt = np.sort(C, axis=1)
    second = srt[:, -2]
    d2 = np.take_along_axis(D, np.argsort(C, axis=1)[:, -2:-1], axis=1)[:, 0]
    clear = (cb - second) > TOL * (db + d2)
    assert np.array_equal(idx[clear], best[clear]), (what, idx, best)
    return int(clear.sum())


@pytest.mark.parametrize("K,N,seed", [(512, 1024, 40), (1152, 608, 41), (5120, 8192, 42)])
def test_argmax_parity(K, N, seed):
    A, qw, sc = synth.gen_problem(K, N, seed)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    C16, D16 = oracle.gemm(A, qw, sc, 16, N, K)
    plans = [None] + [p for p in ALL_PLANS if p.splits == 1][::3]
    for M in (1, 2, 4, 5, 9, 16):
        cases = [p for p in plans if p is None or w4.plan_ok(M, N, K, p)]
        note(f"[argmax] K={K} N={N} M={M}: {len(cases)} plans")
        for p in cases:
            idx, val = w4.gemm_argmax(a[:M].contiguous(), blob, s, N, plan=p)
            torch.cuda.synchronize()
            argmax_check(idx, val, C16[:M], D16[:M], (M, p))


def test_argmax_planted_lm_head_unique_and_tie():
    # lm_head geometry; row m's maximum is planted at column target[m] (its
    # codes follow the signs of A[m], scale 1 against 0.01 elsewhere: a
    # margin of thousands of units); row 0's is planted twice, identically,
    # at two columns of different strips: the lower must win.
    wl = synth.WORKLOADS["lm_head"]
    K, N, M = wl.K, wl.N, 9
    A, qw, sc = synth.gen_workload("lm_head", M)
    qw = qw.copy()
    sc = sc.copy()
    rng = np.random.default_rng(43)
    target = rng.choice(N, size=M, replace=False)
    tie = int(target[0]) + 4096 * 16 + 3              # another strip, same row-0 pattern
    a_val = oracle.bf16_bits_to_f64(A)
    for m, n in list(enumerate(target)) + [(0, tie)]:
        codes = np.where(a_val[m] > 0, 15, 0).astype(np.uint32)       # +7 / -8
        words = np.zeros(K // 8, dtype=np.uint32)
        for j in range(8):
            words |= codes[j::8] << np.uint32(4 * j)
        qw[:, n] = words
        sc[:, n] = 0x3F80
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    note(f"[argmax lm_head] targets={target.tolist()} tie={tie}")
    for Mi in (1, 4, 9):
        for rep in range(2):
            idx, val = w4.gemm_argmax(a[:Mi].contiguous(), blob, s, N)
            torch.cuda.synchronize()
            got = idx.cpu().numpy()
            want = target[:Mi].copy()
            want[0] = min(int(target[0]), tie)
            assert np.array_equal(got, want), (Mi, got, want)
            # the reported value against the oracle at that column
            Cc, Dc = oracle.gemm(A, qw, sc, Mi, N, K, cols=want)
            v = val.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(v - np.diag(Cc)) <= TOL * np.diag(Dc)), (v, np.diag(Cc))


def test_argmax_workspace_shared_with_split_k():
    K, N = 1280, 528
    A, qw, sc = synth.gen_problem(K, N, 44)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    C16, D16 = oracle.gemm(A, qw, sc, 16, N, K)
    split = w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_RING)
    ws = torch.zeros(w4.workspace_bytes(16, N, K, split), dtype=torch.uint8, device=DEV)
    first = None
    for rnd in range(3):
        for M in (3, 16):
            C = run_gemm(a, blob, s, N, M, plan=split, ws=ws)
            assert max_err(C, C16[:M], D16[:M]) <= TOL
            idx, val = w4.gemm_argmax(a[:M].contiguous(), blob, s, N, workspace=ws)
            torch.cuda.synchronize()
            argmax_check(idx, val, C16[:M], D16[:M], (rnd, M))
            if M == 16:
                if first is None:
                    first = (idx.clone(), val.clone())
                assert torch.equal(idx, first[0]) and torch.equal(val, first[1])
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
    with pytest.raises(w4.W4A16Error):
        w4.gemm_argmax(a[:2].contiguous(), blob, s, N, plan=split, workspace=ws)   # splits must be 1


# ------------------------------------------------------------- fp32 output, tensor-parallel shards

@pytest.mark.parametrize("K,N,seed", [(512, 1024, 50), (1152, 592, 51)])
def test_f32_output_parity(K, N, seed):
    A, qw, sc = synth.gen_problem(K, N, seed)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    C16, D16 = oracle.gemm(A, qw, sc, 16, N, K)
    worst = 0.0
    for M in (1, 2, 4, 5, 8, 16):
        cases = [None] + [p for p in ALL_PLANS if w4.plan_ok(M, N, K, p)][::2]
        for p in cases:
            C = w4.gemm_f32(a[:M].contiguous(), blob, s, N, plan=p)
            torch.cuda.synchronize()
            e = oracle.normalized_error(C.cpu().numpy().astype(np.float64), C16[:M], D16[:M])
            worst = max(worst, float(e.max()))
            assert e.max() <= TOL, (M, p, float(e.max()))
            # the bf16 call rounds exactly these sums
            if p is None:
                Cb = run_gemm(a, blob, s, N, M)
                assert torch.equal(Cb, C.to(torch.bfloat16))
    note(f"  fp32 worst normalized error {worst:.3e}")


@pytest.mark.parametrize("tp", [2, 4, 8])
def test_tensor_parallel_row_shards_sum_to_the_full_matmul(tp):
    # down projection geometry along K (17408 = 136 groups), narrow N: each
    # shard holds K/tp rows of W (whole groups) and the matching columns of
    # A; the fp32 shard outputs summed equal the full product within the bound
    K, N = 17408, 512
    A, qw, sc = synth.gen_problem(K, N, 52, act="silu_mul")
    Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K)
    Ki = K // tp
    total = None
    for i in range(tp):
        A_i = np.ascontiguousarray(A[:, i * Ki:(i + 1) * Ki])
        qw_i = np.ascontiguousarray(qw[i * Ki // 8:(i + 1) * Ki // 8])
        sc_i = np.ascontiguousarray(sc[i * Ki // 128:(i + 1) * Ki // 128])
        q, s, a = to_dev(qw_i, sc_i, A_i)
        blob = w4.repack_weights(q, Ki, N)
        C_i = w4.gemm_f32(a, blob, s, N)
        total = C_i if total is None else total + C_i
    torch.cuda.synchronize()
    e = oracle.normalized_error(total.cpu().numpy().astype(np.float64), Cref, Dref)
    note(f"[tp rows] tp={tp} K_i={Ki} worst {e.max():.3e}")
    assert e.max() <= TOL


def test_tensor_parallel_column_shards():
    # QKV geometry split four ways by columns: each shard is the matmul of
    # its columns.  Run with the full matrix's plan, a shard equals those
    # columns of the full product bitwise (the same sums in the same order);
    # with its own (narrower) plan it meets the tolerance against the oracle.
    K, N, tp, M = 5120, 8192, 4, 4
    A, qw, sc = synth.gen_problem(K, N, 53)
    q, s, a = to_dev(qw, sc, A)
    p_full = w4.get_plan(M, N, K)
    full = run_gemm(a, w4.repack_weights(q, K, N), s, N, M, plan=p_full)
    Cref, Dref = oracle.gemm(A, qw, sc, M, N, K)
    Ni = N // tp
    for i in range(tp):
        qw_i = np.ascontiguousarray(qw[:, i * Ni:(i + 1) * Ni])
        sc_i = np.ascontiguousarray(sc[:, i * Ni:(i + 1) * Ni])
        q_i, s_i, _ = to_dev(qw_i, sc_i)
        blob_i = w4.repack_weights(q_i, K, Ni)
        C_i = run_gemm(a, blob_i, s_i, Ni, M, plan=p_full)
        assert torch.equal(C_i, full[:, i * Ni:(i + 1) * Ni]), i
        C_own = run_gemm(a, blob_i, s_i, Ni, M)
        note(f"[tp cols] shard {i}: own plan {w4.get_plan(M, Ni, K).as_dict()}")
        assert max_err(C_own, Cref[:, i * Ni:(i + 1) * Ni], Dref[:, i * Ni:(i + 1) * Ni]) <= TOL, i


# ------------------------------------------------------------- maximum K

def test_gemm_maximum_k():
    # K = 2^24, the largest valid K (131072 groups): A is too long to stage in
    # LDS, so the planner streams it; one 16-column tile
    K, N = 1 << 24, 16
    A, qw, sc = synth.gen_problem(K, N, 51, M=8)
    q, s, a = to_dev(qw, sc, A)
    blob = w4.repack_weights(q, K, N)
    Cref, Dref = oracle.gemm(A, qw, sc, 8, N, K)
    for M in (1, 3, 8):
        note(f"[max K] M={M} plan={w4.get_plan(M, N, K)}")
        C = run_gemm(a, blob, s, N, M)
        e = max_err(C, Cref[:M], Dref[:M])
        assert e <= TOL, (M, e)
