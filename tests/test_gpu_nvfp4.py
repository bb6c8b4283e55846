"""GPU parity of the NVFP4 weight-only variant: the HIP path against the CPU
oracle (oracle/nvfp4.c), through the C ABI.

Bars, as for the GPTQ path:
  * repacked blob and scales, fp32 dequantized weights: bit-exact;
  * C: max over outputs of |C_gpu - C_ref| / (|alpha| sum_k |a_k w_k|) <= 2e-3;
  * inputs whose exact result is representable: bitwise equal to the
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
ALPHA = synth.NVFP4_ALPHA


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(packed, scales, A=None):
    """Device copies: blob and scales repacked by the HIP path, bf16 A."""
    N, K = packed.shape[0], packed.shape[1] * 2
    p = torch.from_numpy(np.ascontiguousarray(packed)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    blob, sc = w4.nvfp4_repack(p, s, K, N)
    a = None if A is None else torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).to(DEV).view(torch.bfloat16)
    return blob, sc, a


def c_bits(C):
    return C.view(torch.int16).cpu().numpy().view(np.uint16)


def run(a, blob, sc, N, M, alpha=ALPHA, plan=None, ws=None):
    out = w4.nvfp4_gemm(a[:M].contiguous(), blob, sc, alpha, N, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    return out


def max_err(C, Cref, Dref):
    return float(oracle.normalized_error(oracle.bf16_bits_to_f64(c_bits(C)), Cref, Dref).max())


ALL_PLANS = []
for path in (w4.PATH_GEMV, w4.PATH_MFMA):
    for t in (1, 2, 4, 8):
        for kw in (1, 2, 4, 8):
            for asrc in ((w4.ASRC_LDS,) if path == w4.PATH_GEMV else (w4.ASRC_LDS, w4.ASRC_GLOBAL, w4.ASRC_RING, w4.ASRC_SPLITN)):
                for depth in (0, 2, 3, 4, 5, 8, 10):
                    ALL_PLANS.append(w4.make_plan(path, t, kw, 1, asrc, depth))


def plans_for(M, N, K):
    return [p for p in ALL_PLANS if w4.nvfp4_plan_ok(M, N, K, p)]


def _any_finite_scales(rng, N, K):
    """Every finite E4M3 byte: subnormal, negative and zero scales included."""
    sc = rng.integers(0, 256, size=(N, K // 16), dtype=np.uint8)
    sc[(sc & 0x7F) == 0x7F] = 0x38
    return sc


# ------------------------------------------------------------- bit-exact weights

@pytest.mark.parametrize("K,N,seed", [(128, 16, 1), (640, 80, 2), (1280, 1040, 3), (5120, 8192, 4)])
def test_nvfp4_repack_and_dequant_bit_exact(K, N, seed):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = _any_finite_scales(rng, N, K)
    blob, sc, _ = to_dev(packed, scales)
    W = w4.nvfp4_dequant(blob, sc, K, N)
    torch.cuda.synchronize()
    assert np.array_equal(blob.cpu().numpy(), oracle.nvfp4_repack(packed, K, N))
    assert np.array_equal(sc.cpu().numpy(), oracle.nvfp4_repack_scales(scales, K, N))
    assert np.array_equal(W.cpu().numpy().astype(np.float64), oracle.nvfp4_dequant(packed, scales, K, N))


# ------------------------------------------------------------- GEMM, all plans

@pytest.mark.parametrize("K,N,seed", [(640, 80, 5), (128, 16, 6), (1280, 272, 7), (512, 1024, 8)])
def test_nvfp4_gemm_parity_every_plan_every_m(K, N, seed):
    A, packed, scales = synth.gen_nvfp4_problem(K, N, seed)
    blob, sc, a = to_dev(packed, scales, A)
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    worst = 0.0
    for M in range(1, 17):
        cases = [None] + plans_for(M, N, K)
        note(f"[nvfp4 gemm] K={K} N={N} M={M}: {len(cases)} plans")
        for p in cases:
            C = run(a, blob, sc, N, M, plan=p)
            e = max_err(C, Cref[:M], Dref[:M])
            worst = max(worst, e)
            assert e <= TOL, (M, p, e)
    note(f"  worst normalized error {worst:.3e}")


def test_nvfp4_gemm_every_scale_byte():
    # subnormal, negative and zero block scales, a negative per-tensor factor
    K, N = 768, 48
    rng = np.random.default_rng(11)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = _any_finite_scales(rng, N, K)
    A = synth.gen_activations(16, K, rng)
    blob, sc, a = to_dev(packed, scales, A)
    alpha = float(np.float32(-0.37))
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, alpha, 16, N, K)
    for M in (1, 2, 4, 7, 16):
        for p in [None] + plans_for(M, N, K):
            C = run(a, blob, sc, N, M, alpha=alpha, plan=p)
            assert max_err(C, Cref[:M], Dref[:M]) <= TOL, (M, p)


@pytest.mark.parametrize("K,N,seed", [(5120, 96, 9), (17408, 48, 10)])
def test_nvfp4_gemm_parity_long_k(K, N, seed):
    A, packed, scales = synth.gen_nvfp4_problem(K, N, seed)
    blob, sc, a = to_dev(packed, scales, A)
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    for M in (1, 2, 4, 5, 16):
        cases = [None] + plans_for(M, N, K)
        note(f"[nvfp4 long K] K={K} N={N} M={M}: {len(cases)} plans")
        for p in cases:
            C = run(a, blob, sc, N, M, plan=p)
            assert max_err(C, Cref[:M], Dref[:M]) <= TOL, (M, p)


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_nvfp4_split_k_parity_and_reuse(splits):
    K, N = 1280, 528
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 21)
    blob, sc, a = to_dev(packed, scales, A)
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    for M in (1, 3, 4, 8, 16):
        for path, asrc in ((w4.PATH_GEMV, 0), (w4.PATH_MFMA, 0), (w4.PATH_MFMA, 1), (w4.PATH_MFMA, 2), (w4.PATH_MFMA, 3)):
            if path == w4.PATH_GEMV and M > 4:
                continue
            for t, kw in ((1, 8), (2, 4)):
                p = w4.make_plan(path, t, kw, splits, asrc)
                if not w4.nvfp4_plan_ok(M, N, K, p):
                    continue
                nbytes = w4.nvfp4_workspace_bytes(M, N, K, p)
                assert nbytes > 0
                ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
                note(f"[nvfp4 split-k] M={M} plan={p}")
                C1 = run(a, blob, sc, N, M, plan=p, ws=ws)
                C2 = run(a, blob, sc, N, M, plan=p, ws=ws)
                assert max_err(C1, Cref[:M], Dref[:M]) <= TOL
                assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
                assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_nvfp4_ring_tail_every_remainder():
    # as for GPTQ: K = 128 * G, one wavefront along K, so every remainder of
    # the ring depth and every "fewer groups than slots" case occurs
    N = 64
    for G in range(1, 12):
        K = 128 * G
        A, packed, scales = synth.gen_nvfp4_problem(K, N, 70 + G)
        blob, sc, a = to_dev(packed, scales, A)
        Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
        ran = 0
        for M in (1, 4, 9):
            for path, asrc in ((w4.PATH_GEMV, w4.ASRC_LDS), (w4.PATH_MFMA, w4.ASRC_LDS), (w4.PATH_MFMA, w4.ASRC_RING)):
                for t, kw in ((1, 1), (2, 1), (1, 4), (2, 4), (1, 8)):
                    for d in (2, 3, 4, 5, 8, 10):
                        p = w4.make_plan(path, t, kw, 1, asrc, d)
                        if not w4.nvfp4_plan_ok(M, N, K, p):
                            continue
                        C1 = run(a, blob, sc, N, M, plan=p)
                        C2 = run(a, blob, sc, N, M, plan=p)
                        assert max_err(C1, Cref[:M], Dref[:M]) <= TOL, (G, M, p)
                        assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), (G, M, p)
                        ran += 1
        note(f"[nvfp4 ring tail] G={G}: {ran} plans")
        assert ran > 0


def test_nvfp4_remainder_split_parity():
    # the leading strips whole, the rest split along K (the automatic NVFP4
    # plans of the down projection at one and two rows and of the gate/up
    # width from five rows): GEMV, staged, ring and split-N strips
    K, N = 2048, 1040
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 22)
    blob, sc, a = to_dev(packed, scales, A)
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    ws = torch.zeros(65536 + 4 * 16 * N * 4, dtype=torch.uint8, device=DEV)
    ran = 0
    for M in (1, 2, 5, 8, 16):
        for (path, t, kw, d, asrc) in ((w4.PATH_GEMV, 1, 8, 2, w4.ASRC_LDS), (w4.PATH_MFMA, 1, 8, 4, w4.ASRC_LDS),
                                       (w4.PATH_MFMA, 1, 4, 4, w4.ASRC_SPLITN), (w4.PATH_MFMA, 2, 4, 2, w4.ASRC_RING)):
            nstrips = -(-(N // 16) // (t * (kw if asrc == w4.ASRC_SPLITN else 1)))
            for S in (2, 4):
                for whole in sorted({1, nstrips // 2, nstrips - 1}):
                    p = w4.make_plan(path, t, kw, S, asrc, d, whole)
                    if not w4.nvfp4_plan_ok(M, N, K, p):
                        continue
                    C1 = run(a, blob, sc, N, M, plan=p, ws=ws)
                    C2 = run(a, blob, sc, N, M, plan=p, ws=ws)
                    assert max_err(C1, Cref[:M], Dref[:M]) <= TOL, (M, p)
                    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), (M, p)
                    ran += 1
    note(f"[nvfp4 remainder split] {ran} plans")
    assert ran >= 30
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


# ------------------------------------------------------------- exact special inputs

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_nvfp4_exact_one_hot_rows_blocks_and_alpha():
    # scale (n, kb) = 2^(e - 7) with e = 1 + (n + kb) % 12; row m of A one-hot
    # at k_m; C[m, n] = alpha * e2m1(code(k_m, n)) * 2^(e - 7), exact in bf16
    K, N = 1024, 48
    rng = np.random.default_rng(12)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    e = (np.arange(N)[:, None] + np.arange(K // 16)[None, :]) % 12 + 1
    scales = (e << 3).astype(np.uint8)
    ks = [0, 3, 15, 16, 17, 127, 128, 129, 255, 300, 511, 512, 777, 896, 1000, 1023]
    A = np.zeros((16, K), dtype=np.uint16)
    for m, k in enumerate(ks):
        A[m, k] = 0x3F80
    blob, sc, a = to_dev(packed, scales, A)
    for alpha in (1.0, 2.0 ** -3):
        expect = np.array([[alpha * E2M1[(int(packed[n, k // 2]) >> (4 * (k % 2))) & 0xF] *
                            2.0 ** (int(e[n, k // 16]) - 7) for n in range(N)] for k in ks])
        ebits = oracle.f32_exact_to_bf16_bits(expect)
        for M in (1, 4, 9, 16):
            for p in [None] + plans_for(M, N, K):
                C = run(a, blob, sc, N, M, alpha=alpha, plan=p)
                got = c_bits(C)
                # -0 and +0 both stand for an exact zero
                same = (got == ebits[:M]) | ((got & 0x7FFF) == 0) & ((ebits[:M] & 0x7FFF) == 0)
                assert np.all(same), (alpha, M, p)


def test_nvfp4_exact_ones_column_sums():
    # A = 1, every scale 1.0, alpha 1: C = the column's sum of E2M1 values,
    # a multiple of 1/2 below 2^15: exact in every partial sum
    K, N = 2048, 64
    rng = np.random.default_rng(13)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x38, dtype=np.uint8)
    A = np.full((16, K), 0x3F80, dtype=np.uint16)
    blob, sc, a = to_dev(packed, scales, A)
    colsum = np.array([sum(E2M1[b & 0xF] + E2M1[b >> 4] for b in packed[n].tolist()) for n in range(N)])
    ebits = oracle.f32_exact_to_bf16_bits(colsum)
    for M in (1, 2, 4, 8, 16):
        for p in [None] + plans_for(M, N, K):
            C = run(a, blob, sc, N, M, alpha=1.0, plan=p)
            got = c_bits(C)
            assert np.all((got == ebits[None, :]) | (((got & 0x7FFF) == 0) & ((ebits[None, :] & 0x7FFF) == 0))), (M, p)


# ------------------------------------------------------------- determinism

def test_nvfp4_determinism_and_row_prefix():
    K, N = 5120, 2048
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 31)
    blob, sc, a = to_dev(packed, scales, A)
    for p in plans_for(16, N, K):
        C16 = run(a, blob, sc, N, 16, plan=p)
        C16b = run(a, blob, sc, N, 16, plan=p)
        assert torch.equal(C16.view(torch.int16), C16b.view(torch.int16)), p
        for M in (5, 8, 9):
            CM = run(a, blob, sc, N, M, plan=p)
            assert torch.equal(CM.view(torch.int16), C16[:M].view(torch.int16)), (M, p)


# ------------------------------------------------------------- full workload sizes

@pytest.mark.parametrize("name", ["qkv", "attn_out", "gate_up", "down"])
def test_nvfp4_workload_parity_full(name):
    wl = synth.WORKLOADS[name]
    K, N = wl.K, wl.N
    Ms = (1, 2, 3, 4, 5, 6, 7, 8, 9, 16)
    note(f"[nvfp4 workload] {name} K={K} N={N} Ms={Ms}")
    A, packed, scales = synth.gen_nvfp4_workload(name)
    blob, sc, a = to_dev(packed, scales, A)
    torch.cuda.synchronize()
    assert np.array_equal(blob.cpu().numpy(), oracle.nvfp4_repack(packed, K, N))
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    for M in Ms:
        C = run(a, blob, sc, N, M)
        e = max_err(C, Cref[:M], Dref[:M])
        note(f"  M={M} plan={w4.nvfp4_get_plan(M, N, K)} max normalized error {e:.3e}")
        assert e <= TOL


def test_nvfp4_workload_parity_lm_head_sampled():
    wl = synth.WORKLOADS["lm_head"]
    K, N = wl.K, wl.N
    A, packed, scales = synth.gen_nvfp4_workload("lm_head")
    blob, sc, a = to_dev(packed, scales, A)
    rng = np.random.default_rng(99)
    cols = np.unique(np.concatenate([rng.integers(0, N, 2000), np.arange(16), np.arange(N - 16, N)]))
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K, cols=cols)
    for M in (1, 8, 16):
        C = run(a, blob, sc, N, M)
        got = oracle.bf16_bits_to_f64(c_bits(C))[:, cols]
        e = float(oracle.normalized_error(got, Cref[:M], Dref[:M]).max())
        note(f"  lm_head M={M} plan={w4.nvfp4_get_plan(M, N, K)} max normalized error {e:.3e}")
        assert e <= TOL


def test_nvfp4_maximum_k():
    # K = 2^24, the largest valid K: A streams (global memory or the ring)
    K, N = 1 << 24, 16
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 52, M=5)
    blob, sc, a = to_dev(packed, scales, A)
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 5, N, K)
    for M in (1, 2, 5):
        note(f"[nvfp4 max K] M={M} plan={w4.nvfp4_get_plan(M, N, K)}")
        C = run(a, blob, sc, N, M)
        assert max_err(C, Cref[:M], Dref[:M]) <= TOL, M
