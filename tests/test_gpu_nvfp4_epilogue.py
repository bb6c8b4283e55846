"""GPU parity of the NVFP4 epilogue modes (gate/up activation, row argmax,
fp32 output), through the C ABI, against the CPU oracle.

The bars are those of the GPTQ epilogues, with every sum scaled by alpha:
  * SiLU(gate) * up: |H - H_ref| <= 2e-3 E + one bf16 rounding of H, E the
    oracle's first-order bound (nvfp4_gemm_silu_mul);
  * argmax: the exact winner wherever the top two are apart by more than
    their bounds, else a column within the bound of the exact maximum; the
    value within the bound of that column's exact sum; planted maxima exact;
  * fp32 output: normalized error <= 2e-3, and the bf16 call rounds exactly
    these sums; K shards summed equal the whole product within the bound.
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
    N, K = packed.shape[0], packed.shape[1] * 2
    p = torch.from_numpy(np.ascontiguousarray(packed)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    blob, sc = w4.nvfp4_repack(p, s, K, N)
    a = None if A is None else torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).to(DEV).view(torch.bfloat16)
    return blob, sc, a


def c_bits(C):
    return C.view(torch.int16).cpu().numpy().view(np.uint16)


ALL_PLANS = []
for path in (w4.PATH_GEMV, w4.PATH_MFMA):
    for t in (1, 2, 4, 8):
        for kw in (1, 2, 4, 8):
            for asrc in ((w4.ASRC_LDS,) if path == w4.PATH_GEMV else (w4.ASRC_LDS, w4.ASRC_GLOBAL, w4.ASRC_RING, w4.ASRC_SPLITN)):
                for depth in (0, 2, 3, 4, 5, 8, 10):
                    ALL_PLANS.append(w4.make_plan(path, t, kw, 1, asrc, depth))
EVEN_PLANS = [p for p in ALL_PLANS if p.tiles % 2 == 0]


# ------------------------------------------------------------- gate/up activation

def silu_mul_check(H, Href, E, what):
    got = oracle.bf16_bits_to_f64(c_bits(H))
    err = np.abs(got - Href)
    # + 2^-100: the activation runs in fp32, where exp(-g) overflows for
    # g < -88.7 and silu(g) becomes -0; the exact |H| there is below
    # 88 e^-88 |u| < 1e-36 |u|, far under this floor for any |u| < 1e6
    bound = TOL * E * 1.01 + 2.0 ** -8 * np.abs(Href) * (1 + 1e-6) + 2.0 ** -100
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float((err - bound).max()))


@pytest.mark.parametrize("K,N,seed,alpha", [(512, 1024, 60, ALPHA), (1152, 608, 61, -0.0625),
                                            (384, 64, 62, ALPHA)])
def test_nvfp4_silu_mul_parity_even_plans(K, N, seed, alpha):
    A, packed, scales = synth.gen_nvfp4_problem(K, N, seed)
    blob, sc, a = to_dev(packed, scales, A)
    Href16, E16 = oracle.nvfp4_gemm_silu_mul(A, packed, scales, alpha, 16, N, K)
    for M in (1, 2, 3, 4, 5, 8, 16):
        cases = [None] + [p for p in EVEN_PLANS if w4.nvfp4_plan_ok(M, N, K, p)][::2]
        note(f"[nvfp4 silu-mul] K={K} N={N} M={M} alpha={alpha}: {len(cases)} plans")
        for p in cases:
            H = w4.nvfp4_gemm_silu_mul(a[:M].contiguous(), blob, sc, alpha, N, plan=p)
            torch.cuda.synchronize()
            silu_mul_check(H, Href16[:M], E16[:M], (M, p))


@pytest.mark.parametrize("splits", [2, 4])
def test_nvfp4_silu_mul_split_k(splits):
    K, N = 1280, 544
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 63)
    blob, sc, a = to_dev(packed, scales, A)
    Href, E = oracle.nvfp4_gemm_silu_mul(A, packed, scales, ALPHA, 16, N, K)
    for M in (1, 4, 9, 16):
        for path, asrc in ((w4.PATH_GEMV, 0), (w4.PATH_MFMA, 0), (w4.PATH_MFMA, 1), (w4.PATH_MFMA, 2), (w4.PATH_MFMA, 3)):
            if path == w4.PATH_GEMV and M > 4:
                continue
            p = w4.make_plan(path, 2, 4, splits, asrc)
            if not w4.nvfp4_plan_ok(M, N, K, p):
                continue
            ws = torch.zeros(w4.nvfp4_workspace_bytes(M, N, K, p), dtype=torch.uint8, device=DEV)
            note(f"[nvfp4 silu-mul split] M={M} plan={p}")
            H1 = w4.nvfp4_gemm_silu_mul(a[:M].contiguous(), blob, sc, ALPHA, N, plan=p, workspace=ws)
            H2 = w4.nvfp4_gemm_silu_mul(a[:M].contiguous(), blob, sc, ALPHA, N, plan=p, workspace=ws)
            torch.cuda.synchronize()
            silu_mul_check(H1, Href[:M], E[:M], (M, p))
            assert torch.equal(H1.view(torch.int16), H2.view(torch.int16))
            assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_nvfp4_silu_mul_zero_gate_is_exact_zero_and_odd_tiles_rejected():
    K, N = 512, 256
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 64)
    packed = packed.copy()
    packed[: N // 2] = 0x80                     # gate codes +0 and -0
    blob, sc, a = to_dev(packed, scales, A)
    for M in (1, 4, 16):
        H = w4.nvfp4_gemm_silu_mul(a[:M].contiguous(), blob, sc, ALPHA, N)
        torch.cuda.synchronize()
        assert int((H.view(torch.int16) & 0x7FFF).abs().sum()) == 0
    with pytest.raises(w4.W4A16Error):
        w4.nvfp4_gemm_silu_mul(a[:1].contiguous(), blob, sc, ALPHA, N, plan=w4.make_plan(w4.PATH_GEMV, 1, 4))


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 2, 4, 8, 9, 16])
def test_nvfp4_silu_mul_gate_up_workload(M):
    wl = synth.WORKLOADS["gate_up"]
    K, N = wl.K, wl.N
    A, packed, scales = synth.gen_nvfp4_workload("gate_up")
    blob, sc, a = to_dev(packed, scales, A)
    js = np.random.default_rng(65).choice(N // 2, size=2048, replace=False)
    Href, E = oracle.nvfp4_gemm_silu_mul(A, packed, scales, ALPHA, M, N, K, js=js)
    H = w4.nvfp4_gemm_silu_mul(a[:M].contiguous(), blob, sc, ALPHA, N)
    torch.cuda.synchronize()
    note(f"[nvfp4 silu-mul gate_up] M={M} plan={w4.nvfp4_get_plan(M, N, K).as_dict()}")
    silu_mul_check(H[:, torch.from_numpy(js).to(DEV)], Href, E, M)


# ------------------------------------------------------------- greedy pick (row argmax)

def argmax_check(idx, val, C, D, what):
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


@pytest.mark.parametrize("K,N,seed", [(512, 1024, 66), (1152, 608, 67), (5120, 8192, 68)])
def test_nvfp4_argmax_parity_both_signs_of_alpha(K, N, seed):
    A, packed, scales = synth.gen_nvfp4_problem(K, N, seed)
    blob, sc, a = to_dev(packed, scales, A)
    plans = [None] + [p for p in ALL_PLANS if p.splits == 1][::5]
    for alpha in (ALPHA, -ALPHA):
        C16, D16 = oracle.nvfp4_gemm(A, packed, scales, alpha, 16, N, K)
        clear = 0                    # rows whose winner is fixed by the bound: some must exist
        for M in (1, 2, 4, 5, 9, 16):
            cases = [p for p in plans if p is None or w4.nvfp4_plan_ok(M, N, K, p)]
            note(f"[nvfp4 argmax] K={K} N={N} M={M} alpha={alpha}: {len(cases)} plans")
            for p in cases:
                idx, val = w4.nvfp4_gemm_argmax(a[:M].contiguous(), blob, sc, alpha, N, plan=p)
                torch.cuda.synchronize()
                clear += argmax_check(idx, val, C16[:M], D16[:M], (M, p, alpha))
        assert clear > 0


def test_nvfp4_argmax_planted_lm_head_unique_and_tie():
    # lm_head geometry; row m's extreme is planted at column target[m]: codes
    # +-6 following the signs of A[m] (reversed for a negative alpha), block
    # scales 448 against at most 8 elsewhere.  Row 0's is planted twice,
    # identically, in two different strips: the lower column must win.
    wl = synth.WORKLOADS["lm_head"]
    K, N, M = wl.K, wl.N, 9
    A, packed, scales = synth.gen_nvfp4_workload("lm_head", M)
    rng = np.random.default_rng(69)
    target = rng.choice(N, size=M, replace=False)
    tie = int(target[0]) + 4096 * 16 + 3
    a_val = oracle.bf16_bits_to_f64(A)
    for alpha in (ALPHA, -ALPHA):
        pk = packed.copy()
        sc = scales.copy()
        for m, n in list(enumerate(target)) + [(0, tie)]:
            pos = (a_val[m] > 0) == (alpha > 0)
            codes = np.where(pos, 7, 15).astype(np.uint8)          # +6 / -6
            pk[n] = codes[0::2] | (codes[1::2] << 4)
            sc[n] = 0x7E                                            # 448
        blob, s, a = to_dev(pk, sc, A)
        note(f"[nvfp4 argmax lm_head] alpha={alpha} targets={target.tolist()} tie={tie}")
        for Mi in (1, 4, 9):
            for rep in range(2):
                idx, val = w4.nvfp4_gemm_argmax(a[:Mi].contiguous(), blob, s, alpha, N)
                torch.cuda.synchronize()
                got = idx.cpu().numpy()
                want = target[:Mi].copy()
                want[0] = min(int(target[0]), tie)
                assert np.array_equal(got, want), (alpha, Mi, got, want)
                Cc, Dc = oracle.nvfp4_gemm(A, pk, sc, alpha, Mi, N, K, cols=want)
                v = val.cpu().numpy().astype(np.float64)
                assert np.all(np.abs(v - np.diag(Cc)) <= TOL * np.diag(Dc)), (v, np.diag(Cc))
        del blob, s


def test_nvfp4_argmax_workspace_shared_with_split_k():
    K, N = 1280, 528
    A, packed, scales = synth.gen_nvfp4_problem(K, N, 70)
    blob, sc, a = to_dev(packed, scales, A)
    C16, D16 = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    split = w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_RING)
    ws = torch.zeros(max(w4.nvfp4_workspace_bytes(16, N, K, split), w4.ARGMAX_WORKSPACE_BYTES),
                     dtype=torch.uint8, device=DEV)
    first = None
    for rnd in range(3):
        for M in (3, 16):
            C = w4.nvfp4_gemm(a[:M].contiguous(), blob, sc, ALPHA, N, plan=split, workspace=ws)
            idx, val = w4.nvfp4_gemm_argmax(a[:M].contiguous(), blob, sc, ALPHA, N, workspace=ws)
            torch.cuda.synchronize()
            e = oracle.normalized_error(oracle.bf16_bits_to_f64(c_bits(C)), C16[:M], D16[:M])
            assert e.max() <= TOL
            argmax_check(idx, val, C16[:M], D16[:M], (rnd, M))
            if M == 16:
                if first is None:
                    first = (idx.clone(), val.clone())
                assert torch.equal(idx, first[0]) and torch.equal(val, first[1])
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
    with pytest.raises(w4.W4A16Error):
        w4.nvfp4_gemm_argmax(a[:2].contiguous(), blob, sc, ALPHA, N, plan=split, workspace=ws)


# ------------------------------------------------------------- fp32 output, tensor-parallel shards

@pytest.mark.parametrize("K,N,seed", [(512, 1024, 71), (1152, 592, 72)])
def test_nvfp4_f32_output_parity(K, N, seed):
    A, packed, scales = synth.gen_nvfp4_problem(K, N, seed)
    blob, sc, a = to_dev(packed, scales, A)
    C16, D16 = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    worst = 0.0
    for M in (1, 2, 4, 5, 8, 16):
        cases = [None] + [p for p in ALL_PLANS if w4.nvfp4_plan_ok(M, N, K, p)][::3]
        for p in cases:
            C = w4.nvfp4_gemm_f32(a[:M].contiguous(), blob, sc, ALPHA, N, plan=p)
            torch.cuda.synchronize()
            e = oracle.normalized_error(C.cpu().numpy().astype(np.float64), C16[:M], D16[:M])
            worst = max(worst, float(e.max()))
            assert e.max() <= TOL, (M, p, float(e.max()))
            if p is None:
                Cb = w4.nvfp4_gemm(a[:M].contiguous(), blob, sc, ALPHA, N)
                torch.cuda.synchronize()
                assert torch.equal(Cb, C.to(torch.bfloat16))
    note(f"  nvfp4 fp32 worst normalized error {worst:.3e}")


@pytest.mark.parametrize("tp", [2, 4, 8])
def test_nvfp4_tensor_parallel_row_shards_sum_to_the_full_matmul(tp):
    # down projection geometry along K, narrow N: shard i holds rows
    # [i K/tp, (i+1) K/tp) of W (whole scale blocks) and those columns of A
    K, N = 17408, 512
    rng = np.random.default_rng(73)
    packed, scales = synth.gen_nvfp4_weights(K, N, rng)
    A = synth.gen_activations(16, K, rng, "silu_mul")
    Cref, Dref = oracle.nvfp4_gemm(A, packed, scales, ALPHA, 16, N, K)
    Ki = K // tp
    total = None
    for i in range(tp):
        A_i = np.ascontiguousarray(A[:, i * Ki:(i + 1) * Ki])
        pk_i = np.ascontiguousarray(packed[:, i * Ki // 2:(i + 1) * Ki // 2])
        sc_i = np.ascontiguousarray(scales[:, i * Ki // 16:(i + 1) * Ki // 16])
        blob, sc, a = to_dev(pk_i, sc_i, A_i)
        C_i = w4.nvfp4_gemm_f32(a, blob, sc, ALPHA, N)
        total = C_i if total is None else total + C_i
    torch.cuda.synchronize()
    e = oracle.normalized_error(total.cpu().numpy().astype(np.float64), Cref, Dref)
    note(f"[nvfp4 tp rows] tp={tp} K_i={Ki} worst {e.max():.3e}")
    assert e.max() <= TOL
