"""The Python binding rejects malformed tensors before any pointer reaches the library.

CPU tensors stand in for device tensors: every check below fires before the
device check (and before any library call), so these run without a GPU.  A
call whose tensors are all well formed but live on the CPU must fail the
device check, never reach the library.
"""
import pytest
import torch

import weight_only_int4_gptq_amd as w4

K, N, M = 512, 1024, 4


def good():
    A = torch.zeros((M, K), dtype=torch.bfloat16)
    blob = torch.zeros(K * N // 2, dtype=torch.uint8)
    scales = torch.zeros((K // 128, N), dtype=torch.bfloat16)
    return A, blob, scales


def nv_good():
    A = torch.zeros((M, K), dtype=torch.bfloat16)
    return A, torch.zeros(K * N // 2, dtype=torch.uint8), torch.zeros(K * N // 16, dtype=torch.uint8)


def bad_cases():
    A, blob, scales = good()
    yield "A dtype", dict(A=A.float())
    yield "A rank", dict(A=torch.zeros(K, dtype=torch.bfloat16))
    yield "A rows", dict(A=torch.zeros((17, K), dtype=torch.bfloat16))
    yield "A K", dict(A=torch.zeros((M, 500), dtype=torch.bfloat16))
    yield "A column slice", dict(A=torch.zeros((M, 2 * K), dtype=torch.bfloat16)[:, :K])
    yield "blob short", dict(blob=blob[:-16])
    yield "blob strided", dict(blob=torch.zeros(K * N, dtype=torch.uint8)[::2])
    yield "scales dtype", dict(scales=scales.float())
    yield "scales shape", dict(scales=torch.zeros((K // 128, N // 2), dtype=torch.bfloat16))
    yield "scales transposed", dict(scales=torch.zeros((N, K // 128), dtype=torch.bfloat16))
    yield "scales strided", dict(scales=torch.zeros((K // 128, 2 * N), dtype=torch.bfloat16)[:, ::2])
    yield "out dtype", dict(out=torch.zeros((M, N), dtype=torch.float32))
    yield "out shape", dict(out=torch.zeros((M, N - 16), dtype=torch.bfloat16))
    yield "out strided", dict(out=torch.zeros((M, 2 * N), dtype=torch.bfloat16)[:, ::2])
    yield "N not a tile multiple", dict(N=1000)
    yield "workspace short", dict(workspace=torch.zeros(100, dtype=torch.uint8))
    yield "plan type", dict(plan="mfma")


@pytest.mark.parametrize("what,kw", list(bad_cases()), ids=[c[0] for c in bad_cases()])
def test_gemm_rejects(what, kw):
    A, blob, scales = good()
    args = dict(A=A, blob=blob, scales=scales, N=N)
    args.update(kw)
    with pytest.raises(ValueError):
        w4.gemm(args.pop("A"), args.pop("blob"), args.pop("scales"), args.pop("N"), **args)


def test_every_wrapper_checks_before_the_library():
    A, blob, scales = good()
    for fn in (w4.gemm, w4.gemm_f32, w4.gemm_silu_mul):
        with pytest.raises(ValueError):
            fn(A.float(), blob, scales, N)
        with pytest.raises(ValueError):
            fn(A, blob[:-1], scales, N)
        with pytest.raises(ValueError):
            fn(A, blob, scales, N, out=torch.zeros((M, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        w4.gemm_argmax(A, blob, scales[:1], N)
    with pytest.raises(ValueError):
        w4.gemm_silu_mul(A, blob, scales, 1008)            # each half must be whole tiles
    with pytest.raises(ValueError):
        w4.dequant_debug(blob, scales[:, :16], K, N)
    with pytest.raises(ValueError):
        w4.unpack_debug(blob[:10], K, N)
    with pytest.raises(ValueError):
        w4.repack_weights(torch.zeros((K // 8, N), dtype=torch.int16), K, N)
    with pytest.raises(ValueError):
        w4.repack_weights(torch.zeros((K // 8, N), dtype=torch.int32), K, N,
                          out=torch.zeros(16, dtype=torch.uint8))
    nA, nblob, nsc = nv_good()
    for fn in (w4.nvfp4_gemm, w4.nvfp4_gemm_f32, w4.nvfp4_gemm_silu_mul):
        with pytest.raises(ValueError):
            fn(nA, nblob, nsc[:-1], 0.5, N)
        with pytest.raises(ValueError):
            fn(nA[:, :256].contiguous(), nblob, nsc, 0.5, N + 16)
    with pytest.raises(ValueError):
        w4.nvfp4_gemm_argmax(nA.float(), nblob, nsc, 0.5, N)
    with pytest.raises(ValueError):
        w4.nvfp4_repack(torch.zeros((N, K // 2 - 1), dtype=torch.uint8), torch.zeros((N, K // 16), dtype=torch.uint8), K, N)


def test_well_formed_host_tensors_fail_the_device_check():
    A, blob, scales = good()
    with pytest.raises(ValueError, match="device"):
        w4.gemm(A, blob, scales, N)
    with pytest.raises(ValueError, match="device"):
        w4.gemm_argmax(A, blob, scales, N)
    nA, nblob, nsc = nv_good()
    with pytest.raises(ValueError, match="device"):
        w4.nvfp4_gemm(nA, nblob, nsc, 0.5, N)
