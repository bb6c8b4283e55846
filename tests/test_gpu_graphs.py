"""Captured calls: a HIP graph of the library's calls replays to the eager results.

Decode and verify steps are replayed from captured graphs, so every kind of
call must be capturable and give, on every replay, bitwise the result of the
same call made eagerly: plain and split-K matmuls (their strip counters are
left at zero by each call), the gate/up activation, the row argmax (its bins
are cleared by the fold kernel) and the NVFP4 calls of every mode.  Between replays the
test runs other eager calls on the same workspaces and synchronizes.
"""
import numpy as np
import pytest
import torch

import synth
import weight_only_int4_gptq_amd as w4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gptq(K, N, seed):
    A, qw, sc = synth.gen_problem(K, N, seed)
    q = torch.from_numpy(qw.view(np.int32)).to(DEV)
    s = torch.from_numpy(sc.view(np.int16)).to(DEV).view(torch.bfloat16)   # the checkpoint's scales
    blob = w4.repack_weights(q, K, N)
    a = torch.from_numpy(A.view(np.int16)).to(DEV).view(torch.bfloat16)
    return a, blob, s


def _nvfp4(K, N, seed):
    A, packed, scales = synth.gen_nvfp4_problem(K, N, seed)
    blob, s = w4.nvfp4_repack(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV), K, N)
    a = torch.from_numpy(A.view(np.int16)).to(DEV).view(torch.bfloat16)
    return a, blob, s


def _same(x, y):
    return torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16)
                       if x.dtype == torch.bfloat16 else x, y.view(torch.int32) if y.dtype == torch.float32
                       else y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_graph_replays_match_eager_calls():
    K, N, M = 1280, 528, 8
    a, blob, s = _gptq(K, N, 41)
    au, blobu, su = _gptq(1024, 1024, 42)                       # gate/up: N = 1024 (two halves of 512)
    al, blobl, sl = _gptq(512, 4096, 43)                        # output projection for the argmax
    an, blobn, sn = _nvfp4(K, N, 44)
    anu, blobnu, snu = _nvfp4(1024, 1024, 45)                   # NVFP4 gate/up
    anl, blobnl, snl = _nvfp4(512, 4096, 46)                    # NVFP4 output projection

    split = w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_LDS)
    nv_split = w4.make_plan(w4.PATH_MFMA, 2, 4, 2, w4.ASRC_RING, 2)
    assert w4.plan_ok(M, N, K, split) and w4.nvfp4_plan_ok(M, N, K, nv_split)
    ws = torch.zeros(max(w4.workspace_bytes(M, N, K, split), 1 << 16), dtype=torch.uint8, device=DEV)
    ws_nv = torch.zeros(w4.nvfp4_workspace_bytes(M, N, K, nv_split), dtype=torch.uint8, device=DEV)
    ws_am = torch.zeros(w4.ARGMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    ws_am_nv = torch.zeros(w4.ARGMAX_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)

    outs = {
        "split": torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
        "auto": torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
        "silu": torch.empty((M, 512), dtype=torch.bfloat16, device=DEV),
        "nv": torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
        "f32": torch.empty((M, N), dtype=torch.float32, device=DEV),
        "nv_silu": torch.empty((M, 512), dtype=torch.bfloat16, device=DEV),
        "nv_f32": torch.empty((M, N), dtype=torch.float32, device=DEV),
    }
    nv_am = {}

    def step():
        w4.gemm(a[:M].contiguous(), blob, s, N, out=outs["split"], plan=split, workspace=ws)
        w4.gemm(a[:M].contiguous(), blob, s, N, out=outs["auto"])
        w4.gemm_silu_mul(au[:M].contiguous(), blobu, su, 1024, out=outs["silu"])
        w4.gemm_f32(a[:M].contiguous(), blob, s, N, out=outs["f32"], plan=split, workspace=ws)
        w4.nvfp4_gemm(an[:M].contiguous(), blobn, sn, synth.NVFP4_ALPHA, N, out=outs["nv"], plan=nv_split,
                      workspace=ws_nv)
        w4.nvfp4_gemm_silu_mul(anu[:M].contiguous(), blobnu, snu, synth.NVFP4_ALPHA, 1024, out=outs["nv_silu"])
        w4.nvfp4_gemm_f32(an[:M].contiguous(), blobn, sn, synth.NVFP4_ALPHA, N, out=outs["nv_f32"],
                          plan=nv_split, workspace=ws_nv)
        nv_am["r"] = w4.nvfp4_gemm_argmax(anl[:M].contiguous(), blobnl, snl, -synth.NVFP4_ALPHA, 4096,
                                          workspace=ws_am_nv)
        return w4.gemm_argmax(al[:M].contiguous(), blobl, sl, 4096, workspace=ws_am)

    # eager reference
    idx0, val0 = step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref_idx, ref_val = idx0.clone(), val0.clone()
    ref_nv_idx, ref_nv_val = (t.clone() for t in nv_am["r"])

    # warm once on the capture stream, then capture
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        gidx, gval = step()
    gnv_idx, gnv_val = nv_am["r"]
    torch.cuda.synchronize()

    for rep in range(3):
        for v in outs.values():
            v.fill_(0)
        gidx.fill_(-1)
        gnv_idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert _same(outs[k], ref[k]), (rep, k)
        assert torch.equal(gidx, ref_idx) and torch.equal(gval.view(torch.int32), ref_val.view(torch.int32)), rep
        assert torch.equal(gnv_idx, ref_nv_idx), rep
        assert torch.equal(gnv_val.view(torch.int32), ref_nv_val.view(torch.int32)), rep
        # eager calls on the same workspaces between replays
        e_idx, _ = step()
        torch.cuda.synchronize()
        assert torch.equal(e_idx, ref_idx)
        for k in outs:
            assert _same(outs[k], ref[k]), (rep, "eager", k)
        # every call left the counter regions zero
        assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
        assert int(ws_nv[:65536].view(torch.int32).abs().sum()) == 0
        assert int(ws_am.view(torch.int64).abs().sum()) == 0
        assert int(ws_am_nv.view(torch.int64).abs().sum()) == 0
