"""The allocation-free matmul call against the call that takes a workspace.

w4a16_gemm_noalloc keeps its split-K counters and partials in a static device
array instead of a caller's workspace.  Through the C ABI, it must give
bitwise the output of w4a16_gemm_plan with the same plan and a zero-filled
workspace, on consecutive calls of decreasing size (the array keeps the
previous call's contents), and reject a plan whose workspace exceeds it.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_int4_gptq_amd as w4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH = 65536 + (4 << 20)          # W4A16_NOALLOC_SCRATCH_BYTES


def lib():
    L = w4.lib()
    P, I = ctypes.c_void_p, ctypes.c_int
    L.w4a16_gemm_noalloc.argtypes = [P, P, P, P, I, I, I, I, ctypes.POINTER(w4.Plan), P]
    L.w4a16_gemm_noalloc.restype = I
    return L


def problem(K, N, seed, act="normal"):
    A, qw, sc = synth.gen_problem(K, N, seed, act)
    a = torch.from_numpy(A.view(np.int16)).to(DEV).view(torch.bfloat16)
    blob = w4.repack_weights(torch.from_numpy(qw.view(np.int32)).to(DEV), K, N)
    s = torch.from_numpy(sc.view(np.int16)).to(DEV).view(torch.bfloat16)
    Cref, Dref = oracle.gemm(A, qw, sc, 16, N, K)
    return a, blob, s, Cref, Dref


def noalloc(a, blob, s, N, M, plan):
    K = a.shape[1]
    C = torch.full((M, N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    st = lib().w4a16_gemm_noalloc(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(blob.data_ptr()),
                                  ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(C.data_ptr()), M, N, K, 128,
                                  ctypes.byref(plan) if plan is not None else None,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, C


def with_workspace(a, blob, s, N, M, plan):
    K = a.shape[1]
    p = plan if plan is not None else w4.get_plan(M, N, K)
    ws = torch.zeros(max(w4.workspace_bytes(M, N, K, p), 16), dtype=torch.uint8, device=DEV)
    C = w4.gemm(a[:M].contiguous(), blob, s, N, plan=p, workspace=ws)
    torch.cuda.synchronize()
    return C


def test_noalloc_automatic_plan_too_large_for_the_array_runs_unsplit():
    # a gate/up-width call at 8 rows: the automatic plan splits the strips
    # beyond two per CU four ways, and those partials (4.5 MB) exceed the
    # array; without a plan the call runs the same plan with every strip
    # whole, bitwise equal to the workspace call with that plan
    K, N, M = 4096, 34816, 8
    A, qw, sc = synth.gen_problem(K, N, 31)
    a = torch.from_numpy(A.view(np.int16)).to(DEV).view(torch.bfloat16)
    blob = w4.repack_weights(torch.from_numpy(qw.view(np.int32)).to(DEV), K, N)
    s = torch.from_numpy(sc.view(np.int16)).to(DEV).view(torch.bfloat16)
    auto = w4.get_plan(M, N, K)
    assert auto.splits > 1 and w4.workspace_bytes(M, N, K, auto) > SCRATCH
    whole = w4.make_plan(auto.path, auto.tiles, auto.kwaves, 1, auto.asrc, auto.depth, 0)
    st, C = noalloc(a[:M].contiguous(), blob, s, N, M, None)
    assert st == 0, w4.status_string(st)
    ref = with_workspace(a, blob, s, N, M, whole)
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16))
    cols = np.arange(0, N, 97, dtype=np.int32)
    Cref, Dref = oracle.gemm(A, qw, sc, M, N, K, cols=cols)
    got = oracle.bf16_bits_to_f64(C.view(torch.int16).cpu().numpy().view(np.uint16))[:, cols]
    assert float(oracle.normalized_error(got, Cref, Dref).max()) <= 2e-3
    # an explicit split plan of that size is still rejected
    st, _ = noalloc(a[:M].contiguous(), blob, s, N, M, auto)
    assert st == -5


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    cases = []
    # the down projection at 8 rows: the automatic plan splits 64 of its
    # strips four ways (655 KiB of partials in the scratch array)
    a, blob, s, Cref, Dref = problem(17408, 5120, 3, "silu_mul")
    assert w4.workspace_bytes(8, 5120, 17408, w4.get_plan(8, 5120, 17408)) > 65536
    cases.append((a, blob, s, Cref, Dref, 5120, 8, None))
    # then a smaller call with an explicit split: fewer strips and rows, so
    # the array holds the previous call's partials beyond what this one writes
    a2, blob2, s2, Cref2, Dref2 = problem(1280, 528, 21)
    cases.append((a2, blob2, s2, Cref2, Dref2, 528, 3, w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_LDS)))
    cases.append((a2, blob2, s2, Cref2, Dref2, 528, 1, w4.make_plan(w4.PATH_GEMV, 1, 4, 2, w4.ASRC_LDS, 0, 10)))
    for rnd in range(2):
        for (a, blob, s, Cref, Dref, N, M, plan) in cases:
            st, C = noalloc(a[:M].contiguous(), blob, s, N, M, plan)
            assert st == 0, (rnd, N, M, w4.status_string(st))
            ref = with_workspace(a, blob, s, N, M, plan)
            assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), (rnd, N, M, plan)
            got = oracle.bf16_bits_to_f64(C.view(torch.int16).cpu().numpy().view(np.uint16))
            assert float(oracle.normalized_error(got, Cref[:M], Dref[:M]).max()) <= 2e-3, (rnd, N, M)


def test_noalloc_rejects_a_plan_beyond_the_scratch_array_and_bad_arguments():
    N, K = 16384, 1024
    a, blob, s, _, _ = problem(K, N, 7)
    big = w4.make_plan(w4.PATH_MFMA, 2, 4, 8, w4.ASRC_LDS)          # 64 KiB + 8 * 16 * 16384 * 4 B
    assert w4.workspace_bytes(16, N, K, big) > SCRATCH
    st, C = noalloc(a[:16].contiguous(), blob, s, N, 16, big)
    assert st == -5                                                     # W4A16_ERR_WORKSPACE
    assert int((C.view(torch.int16) != -1).sum()) == 0                  # nothing ran
    L = lib()
    assert L.w4a16_gemm_noalloc(None, ctypes.c_void_p(blob.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                ctypes.c_void_p(C.data_ptr()), 16, N, K, 128, None, None) == -1
    assert L.w4a16_gemm_noalloc(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(blob.data_ptr()),
                                ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(C.data_ptr()), 16, N, K, 64,
                                None, None) == -3
