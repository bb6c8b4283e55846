"""C-ABI checks that need no GPU: exported symbols, argument validation, planning.

Every error here is raised by the host-side checks before any device work,
so these run on a machine without a GPU.  Compute calls are not made.
"""
import ctypes
import os
import re

import pytest

import weight_only_int4_gptq_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

# fake, 16-byte aligned "device" addresses: never dereferenced, because every
# call below fails its argument checks first
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
ODD = ctypes.c_void_p(0x10008)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    lib = w4.lib()
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(-8, 1):
        s = w4.status_string(st)
        assert s and s != "unknown status"
    assert w4.status_string(-99) == "unknown status"


def test_repacked_bytes():
    assert w4.repacked_bytes(5120, 8192) == 5120 * 8192 // 2
    assert w4.repacked_bytes(100, 16) == 0
    assert w4.repacked_bytes(128, 8) == 0


def _gemm(A=P, wq=P, s=P, C=P2, M=1, N=1024, K=512, group=128, ws=NULL, wsb=0, plan=None):
    L = w4.lib()
    if plan is None:
        return L.w4a16_gemm(A, wq, s, C, M, N, K, group, ws, wsb, NULL)
    return L.w4a16_gemm_plan(A, wq, s, C, M, N, K, group, ws, wsb, ctypes.byref(plan), NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(A=NULL), -1), (dict(wq=NULL), -1), (dict(s=NULL), -1), (dict(C=NULL), -1),
    (dict(M=0), -2), (dict(M=17), -2), (dict(K=500), -2), (dict(K=0), -2), (dict(N=1000), -2),
    (dict(K=(1 << 24) + 128), -2),
    (dict(N=-16), -2), (dict(group=64), -3), (dict(A=ODD), -4), (dict(C=ODD), -4),
    (dict(s=ODD), -4), (dict(wq=ODD), -4),
])
def test_gemm_argument_errors(kw, status):
    assert _gemm(**kw) == status


def test_gemm_plan_errors():
    bad = [
        w4.make_plan(w4.PATH_GEMV, 1, 4),             # GEMV for M > 4
        w4.make_plan(3, 1, 4),                        # unknown path
        w4.make_plan(w4.PATH_MFMA, 3, 4),             # no such tile count
        w4.make_plan(w4.PATH_MFMA, 1, 5),             # no such wave count
        w4.make_plan(w4.PATH_MFMA, 1, 4, splits=0),
        w4.make_plan(w4.PATH_MFMA, 1, 4, splits=8),   # more splits than K groups (K=512)
        w4.make_plan(w4.PATH_MFMA, 1, 4, splits=3),   # not a power of two
        w4.make_plan(w4.PATH_MFMA, 1, 4, asrc=7),
    ]
    for p in bad:
        assert _gemm(M=8, plan=p) == -8, p


def test_remainder_split_plans_are_checked():
    N, K = 1024, 1280                                # 64 one-tile strips, 10 groups
    ok = w4.make_plan(w4.PATH_GEMV, 1, 4, 2, w4.ASRC_LDS, 0, 40)
    assert w4.plan_ok(1, N, K, ok)
    assert w4.plan_ok(1, N, K, w4.make_plan(w4.PATH_GEMV, 1, 4, 2, w4.ASRC_LDS, 0, 64))   # nothing left to split
    assert not w4.plan_ok(1, N, K, w4.make_plan(w4.PATH_GEMV, 1, 4, 2, w4.ASRC_LDS, 0, 65))
    assert not w4.plan_ok(1, N, K, w4.make_plan(w4.PATH_GEMV, 1, 4, 2, w4.ASRC_LDS, 0, -1))
    # the workspace of a remainder split is that of the plain split
    plain = w4.make_plan(w4.PATH_GEMV, 1, 4, 2, w4.ASRC_LDS)
    assert w4.workspace_bytes(1, N, K, ok) == w4.workspace_bytes(1, N, K, plain) == 65536 + 2 * N * 4


def test_split_plan_needs_workspace():
    p = w4.make_plan(w4.PATH_MFMA, 1, 4, splits=2)
    need = w4.workspace_bytes(8, 1024, 512, p)
    assert need == 65536 + 2 * 8 * 1024 * 4
    assert _gemm(M=8, plan=p) == -5
    assert _gemm(M=8, plan=p, ws=P, wsb=need - 1) == -5
    L = w4.lib()
    # short K: the automatic plan does not split (no workspace), but the
    # any-call query still covers the argmax call's counter region
    assert L.w4a16_workspace_bytes_plan(8, 1024, 512, None) == 0
    assert w4.workspace_bytes(8, 1024, 512) == 65536
    for (M, N, K) in ((1, 5120, 17408), (6, 5120, 17408), (16, 8192, 5120), (9, 34816, 5120)):
        auto = L.w4a16_workspace_bytes_plan(M, N, K, None)
        assert w4.workspace_bytes(M, N, K) >= max(auto, 65536), (M, N, K)
    assert L.w4a16_workspace_bytes(0, 1024, 512) == 0


def test_no_device_is_an_error_not_a_crash():
    # valid arguments: on a machine without a gfx950 GPU the device check fails
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _gemm() == -6
    assert w4.lib().w4a16_repack_weights(P, P2, 512, 1024, NULL) == -6
    assert w4.lib().w4a16_dequant_debug(P, P, P2, 512, 1024, NULL) == -6


def test_repack_and_export_argument_errors():
    L = w4.lib()
    assert L.w4a16_repack_weights(NULL, P, 512, 1024, NULL) == -1
    assert L.w4a16_repack_weights(P, P2, 500, 1024, NULL) == -2
    assert L.w4a16_repack_weights(P, P2, 512, 1000, NULL) == -2
    assert L.w4a16_repack_weights(ODD, P2, 512, 1024, NULL) == -4
    assert L.w4a16_dequant_debug(P, NULL, P2, 512, 1024, NULL) == -1
    assert L.w4a16_dequant_debug(P, ODD, P2, 512, 1024, NULL) == -4
    assert L.w4a16_unpack_debug(P, NULL, 512, 1024, NULL) == -1
    assert L.w4a16_unpack_debug(P, P2, 512, 1000, NULL) == -2


def test_boundary_names_of_the_contract():
    # the calls the contract fixes: a one-time weight repack and the matmul on
    # the checkpoint's [K/128, N] scales, plus sizes, the workspace query, the
    # dequant debug export and the status text
    text = open(HEADER).read()
    for sig in (r"size_t\s+w4a16_repacked_bytes\(int K, int N\)",
                r"int\s+w4a16_repack_weights\(const void \*qweight, void \*wq_repacked, int K, int N, void \*stream\)",
                r"size_t\s+w4a16_workspace_bytes\(int M, int N, int K\)",
                r"int\s+w4a16_gemm\(const void \*A, const void \*wq_repacked, const void \*scales, void \*C,\s+"
                r"int M, int N, int K, int group, void \*workspace, size_t workspace_bytes,\s+void \*stream\)",
                r"int\s+w4a16_dequant_debug\(const void \*wq_repacked, const void \*scales, float \*W, int K, int N,",
                r"const char \*w4a16_status_string\(int status\)"):
        assert re.search(sig, text), sig
    L = w4.lib()
    for name in ("w4a16_repacked_bytes", "w4a16_repack_weights", "w4a16_workspace_bytes", "w4a16_gemm",
                 "w4a16_dequant_debug", "w4a16_status_string"):
        assert hasattr(L, name), name
    # scales are consumed as the checkpoint stores them: no scale repack exists
    assert "w4a16_repack_scales(" not in text
    assert not hasattr(L, "w4a16_repack_scales")


def test_row_count_dispatch():
    # one row: the dot2 GEMV kernel; two and more: matrix cores
    for M in range(1, 17):
        p = w4.get_plan(M, 34816, 5120)
        assert p.path == (w4.PATH_GEMV if M == 1 else w4.PATH_MFMA), (M, p)
        # gate/up width: one tile and eight shallow wavefronts at one row;
        # A through the LDS ring from two to 4 rows, two tiles; from five
        # rows four wavefronts split the columns (one tile each up to 8 rows,
        # two above) around a shared ring of depth 4, and the 32 (16) strips
        # beyond two (one) per CU are split four ways along K
        if M == 1:
            assert (p.tiles, p.kwaves, p.depth, p.splits) == (1, 8, 2, 1), (M, p)
        elif M <= 4:
            assert p.asrc == w4.ASRC_RING and p.tiles == 2 and p.splits == 1, (M, p)
        elif M <= 8:
            assert p.asrc == w4.ASRC_SPLITN and (p.tiles, p.kwaves, p.depth, p.splits, p.whole) == (1, 4, 4, 4, 512), (M, p)
        else:
            assert p.asrc == w4.ASRC_SPLITN and (p.tiles, p.kwaves, p.depth, p.splits, p.whole) == (2, 4, 4, 4, 256), (M, p)
    # QKV and attention-out widths (one to two two-tile strips per CU, 40 and
    # 48 groups): eight wavefronts, two tiles, A through the ring, depth 2
    for N, K in ((8192, 5120), (5120, 6144)):
        for M in range(2, 17):
            p = w4.get_plan(M, N, K)
            assert (p.path, p.tiles, p.kwaves, p.splits) == (w4.PATH_MFMA, 2, 8, 1), (N, M, p)
            assert (p.asrc, p.depth) == (w4.ASRC_RING, 2), (N, M, p)
    # very wide N: LDS A at 3-4 rows, the ring at 2, split-N from 5 rows
    # (two tiles per wavefront up to 8 rows, four above)
    assert w4.get_plan(4, 248320, 5120).asrc == w4.ASRC_LDS
    assert w4.get_plan(2, 248320, 5120).asrc == w4.ASRC_RING
    assert w4.get_plan(8, 248320, 5120).asrc == w4.ASRC_SPLITN
    assert w4.get_plan(8, 248320, 5120).tiles == 2
    assert w4.get_plan(16, 248320, 5120).tiles == 4
    # the same for NVFP4 weights from 5 rows; the gate/up width from 5 rows
    # with its strips beyond two per CU split four ways along K
    assert w4.nvfp4_get_plan(5, 248320, 5120).asrc == w4.ASRC_SPLITN
    for M in (5, 8, 9, 16):
        p = w4.nvfp4_get_plan(M, 34816, 5120)
        assert (p.asrc, p.tiles, p.splits, p.whole) == (w4.ASRC_SPLITN, 1, 4, 512), (M, p)
    # NVFP4 down projection: the remainder split at one and two rows; from
    # five rows split-N with every strip in eight K pieces
    for M in (1, 2):
        p = w4.nvfp4_get_plan(M, 5120, 17408)
        assert (p.tiles, p.kwaves, p.splits, p.whole) == (1, 8, 4, 256), (M, p)
    for M in (5, 8, 16):
        p = w4.nvfp4_get_plan(M, 5120, 17408)
        assert (p.asrc, p.tiles, p.kwaves, p.splits, p.depth, p.whole) == (w4.ASRC_SPLITN, 1, 4, 8, 4, 0), (M, p)
    # NVFP4 gate/up width at two to four rows: four-tile strips with A in
    # LDS, the 32 strips beyond two per CU in eight K pieces
    for M in (2, 3, 4):
        p = w4.nvfp4_get_plan(M, 34816, 5120)
        assert (p.asrc, p.tiles, p.kwaves, p.splits, p.depth, p.whole) == (w4.ASRC_LDS, 4, 4, 8, 2, 512), (M, p)
    # NVFP4 QKV and attention-out widths at five and six rows: one tile,
    # eight wavefronts, A in LDS
    for N, K in ((8192, 5120), (5120, 6144)):
        for M in (5, 6):
            p = w4.nvfp4_get_plan(M, N, K)
            assert (p.asrc, p.tiles, p.kwaves, p.splits) == (w4.ASRC_LDS, 1, 8, 1), (N, M, p)
    p = w4.nvfp4_get_plan(1, 34816, 5120)
    assert (p.path, p.tiles, p.kwaves, p.depth) == (w4.PATH_GEMV, 1, 8, 2), p
    p = w4.nvfp4_get_plan(8, 5120, 6144)
    assert (p.asrc, p.tiles, p.kwaves, p.depth) == (w4.ASRC_LDS, 2, 8, 4), p
    # the down projection (320 tiles, 136 groups) at one row and from three
    # to twelve: 256 whole one-tile strips and 64 strips in four K pieces,
    # eight wavefronts, ring depth 4 from three to eight rows; two rows keep
    # the whole K of A in LDS, unsplit; from 13 rows split-N (four one-tile
    # wavefronts around a shared ring of A) with every strip in eight K
    # pieces of 17 groups
    p = w4.get_plan(2, 5120, 17408)
    assert (p.splits, p.asrc, p.tiles, p.kwaves) == (1, w4.ASRC_LDS, 2, 8), p
    for M in (1, 3, 4, 5, 8, 9, 12):
        p = w4.get_plan(M, 5120, 17408)
        assert (p.tiles, p.kwaves, p.splits, p.whole) == (1, 8, 4, 256), (M, p)
        assert p.path == (w4.PATH_GEMV if M == 1 else w4.PATH_MFMA), (M, p)
        assert M == 1 or p.asrc == w4.ASRC_RING, (M, p)
        assert p.depth == (4 if 3 <= M <= 8 else 2), (M, p)
    for M in (13, 16):
        p = w4.get_plan(M, 5120, 17408)
        assert (p.path, p.asrc, p.tiles, p.kwaves, p.depth, p.splits, p.whole) == \
            (w4.PATH_MFMA, w4.ASRC_SPLITN, 1, 4, 4, 8, 0), (M, p)
    # one GPU's tensor-parallel shares at 8 rows: up to 256 tiles, one tile
    # and eight wavefronts with A through the ring; the 544/1088-tile column
    # shards split their strips beyond a whole number per CU four ways; the
    # 68-group K shard of down takes the remainder split like down
    p = w4.get_plan(8, 4096, 5120)
    assert (p.asrc, p.tiles, p.kwaves, p.depth, p.splits) == (w4.ASRC_RING, 1, 8, 4, 1), p
    p = w4.get_plan(8, 17408, 5120)
    assert (p.asrc, p.tiles, p.splits, p.whole) == (w4.ASRC_RING, 2, 4, 512), p
    p = w4.get_plan(8, 8704, 5120)
    assert (p.asrc, p.tiles, p.splits, p.whole) == (w4.ASRC_RING, 2, 4, 256), p
    p = w4.get_plan(8, 5120, 8704)
    assert (p.tiles, p.kwaves, p.splits, p.whole) == (1, 8, 4, 256), p
    p = w4.get_plan(8, 5120, 2176)
    assert (p.asrc, p.tiles, p.depth) == (w4.ASRC_RING, 2, 4), p
    # a K shard of it (68 groups) and the attention output (48 groups) are not split
    assert w4.get_plan(1, 5120, 8704).splits == 1
    assert w4.get_plan(1, 5120, 6144).splits == 1
    assert w4.get_plan(1, 248320, 5120).tiles == 2
    # tiny K: no more K waves than K groups
    assert w4.get_plan(1, 1024, 512).kwaves <= 4
    assert w4.get_plan(1, 1024, 256).kwaves == 1
    for M in range(1, 17):
        for K in (128, 256, 512, 5120, 17408, 1 << 20, 1 << 24):
            for N in (16, 1024, 8192, 34816) + ((131072,) if K <= 5120 else ()):
                if (K // 128) * N * 2 >= 1 << 31:       # scales beyond 32-bit byte offsets
                    assert w4.lib().w4a16_get_plan(M, N, K, ctypes.byref(w4.Plan())) == -2
                    continue
                assert w4.plan_ok(M, N, K, w4.get_plan(M, N, K)), (M, N, K)
                assert w4.nvfp4_plan_ok(M, N, K, w4.nvfp4_get_plan(M, N, K)), (M, N, K)
    p = w4.Plan()
    assert w4.lib().w4a16_get_plan(0, 1024, 512, ctypes.byref(p)) == -2


def test_split_plan_strip_limit():
    # split plans keep one counter per column strip in a fixed 64 KiB region
    ok = w4.make_plan(w4.PATH_MFMA, 1, 4, 2, w4.ASRC_GLOBAL)
    assert w4.plan_ok(8, 16384 * 16, 5120, ok)
    assert not w4.plan_ok(8, 16385 * 16, 5120, ok)
    assert w4.plan_ok(8, 16385 * 16, 5120, w4.make_plan(w4.PATH_MFMA, 2, 4, 2, w4.ASRC_GLOBAL))
    assert w4.plan_ok(8, 16385 * 16, 5120, w4.make_plan(w4.PATH_MFMA, 1, 4, 1, w4.ASRC_GLOBAL))


def test_check_plan():
    ok = w4.make_plan(w4.PATH_MFMA, 1, 8, 1, w4.ASRC_GLOBAL)
    assert w4.plan_ok(16, 34816, 5120, ok)
    # staging 16 rows of K=5120 in LDS does not fit one workgroup's budget
    assert not w4.plan_ok(16, 34816, 5120, w4.make_plan(w4.PATH_MFMA, 1, 8, 1, w4.ASRC_LDS))
    assert w4.plan_ok(16, 34816, 5120, w4.make_plan(w4.PATH_MFMA, 1, 8, 4, w4.ASRC_LDS))
    assert w4.lib().w4a16_check_plan(0, 16, 128, ctypes.byref(ok)) == -2


def _silu_mul(A=P, wq=P, s=P, H=P2, M=1, N=1024, K=512, group=128, ws=NULL, wsb=0, plan=None):
    L = w4.lib()
    if plan is None:
        return L.w4a16_gemm_silu_mul(A, wq, s, H, M, N, K, group, ws, wsb, NULL)
    return L.w4a16_gemm_silu_mul_plan(A, wq, s, H, M, N, K, group, ws, wsb, ctypes.byref(plan), NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(A=NULL), -1), (dict(H=NULL), -1), (dict(M=0), -2), (dict(M=17), -2),
    (dict(N=1008), -2),            # a multiple of 16 but not of 32: halves are not whole tiles
    (dict(K=500), -2), (dict(group=64), -3), (dict(H=ODD), -4),
    (dict(plan=w4.make_plan(w4.PATH_MFMA, 1, 4)), -8),       # odd tile count: no gate/up pairs
])
def test_silu_mul_argument_errors(kw, status):
    assert _silu_mul(**kw) == status


def test_silu_mul_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _silu_mul() == -6
    assert _silu_mul(plan=w4.make_plan(w4.PATH_MFMA, 2, 4)) == -6


def _argmax(A=P, wq=P, s=P, idx=P2, val=P2, M=1, N=1008, K=512, group=128, ws=P, wsb=65536, plan=None):
    L = w4.lib()
    if plan is None:
        return L.w4a16_gemm_argmax(A, wq, s, idx, val, M, N, K, group, ws, wsb, NULL)
    return L.w4a16_gemm_argmax_plan(A, wq, s, idx, val, M, N, K, group, ws, wsb, ctypes.byref(plan), NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(idx=NULL), -1), (dict(val=NULL), -1), (dict(A=NULL), -1), (dict(M=17), -2), (dict(N=1000), -2),
    (dict(group=64), -3), (dict(idx=ctypes.c_void_p(0x20002)), -4),
    (dict(wsb=65535), -5), (dict(ws=NULL), -5),
    (dict(plan=w4.make_plan(w4.PATH_MFMA, 1, 4, 2)), -8),      # splits must be 1
])
def test_argmax_argument_errors(kw, status):
    assert _argmax(**kw) == status


def test_argmax_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _argmax() == -6          # N = 1008: a multiple of 16 is enough here


def _nv(A=P, wq=P, s=P, C=P2, M=1, N=1024, K=512, group=16, ws=NULL, wsb=0, plan=None, alpha=1.0):
    L = w4.lib()
    if plan is None:
        return L.w4a16_nvfp4_gemm(A, wq, s, alpha, C, M, N, K, group, ws, wsb, NULL)
    return L.w4a16_nvfp4_gemm_plan(A, wq, s, alpha, C, M, N, K, group, ws, wsb, ctypes.byref(plan), NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(A=NULL), -1), (dict(C=NULL), -1), (dict(s=NULL), -1), (dict(M=0), -2), (dict(M=17), -2),
    (dict(K=520), -2), (dict(N=1000), -2), (dict(group=128), -3), (dict(C=ODD), -4),
    (dict(plan=w4.make_plan(w4.PATH_MFMA, 1, 1, 1, w4.ASRC_RING)), -8),     # no such NVFP4 ring shape
    (dict(plan=w4.make_plan(w4.PATH_GEMV, 1, 4), M=5), -8),
])
def test_nvfp4_argument_errors(kw, status):
    assert _nv(**kw) == status


def test_nvfp4_sizes_plans_and_no_device():
    assert w4.nvfp4_repacked_bytes(5120, 8192) == 5120 * 8192 // 2
    assert w4.nvfp4_repacked_scale_bytes(5120, 8192) == 5120 * 8192 // 16
    assert w4.nvfp4_repacked_bytes(100, 16) == 0
    L = w4.lib()
    assert L.w4a16_nvfp4_repack_weights(NULL, P, 512, 1024, NULL) == -1
    assert L.w4a16_nvfp4_repack_weights(P, P2, 512, 1000, NULL) == -2
    assert L.w4a16_nvfp4_repack_scales(ODD, P2, 512, 1024, NULL) == -4
    assert L.w4a16_nvfp4_dequant(P, NULL, P2, 512, 1024, NULL) == -1
    for M in range(1, 17):
        for (N, K) in ((8192, 5120), (34816, 5120), (5120, 17408), (248320, 5120), (1024, 512), (16, 128)):
            p = w4.nvfp4_get_plan(M, N, K)
            assert w4.nvfp4_plan_ok(M, N, K, p), (M, N, K, p)
    import torch
    if not torch.cuda.is_available():
        assert _nv() == -6
        assert L.w4a16_nvfp4_repack_weights(P, P2, 512, 1024, NULL) == -6


def _nv_epi(kind, A=P, wq=P, s=P, out=P2, val=P2, M=1, N=1024, K=512, group=16, ws=P, wsb=1 << 24,
            plan=None, alpha=0.5):
    L = w4.lib()
    name = {"silu": "w4a16_nvfp4_gemm_silu_mul", "argmax": "w4a16_nvfp4_gemm_argmax",
            "f32": "w4a16_nvfp4_gemm_f32"}[kind]
    head = (A, wq, s, alpha, out, val) if kind == "argmax" else (A, wq, s, alpha, out)
    tail = (M, N, K, group, ws, wsb)
    if plan is None:
        return getattr(L, name)(*head, *tail, NULL)
    return getattr(L, name + "_plan")(*head, *tail, ctypes.byref(plan), NULL)


@pytest.mark.parametrize("kind,kw,status", [
    ("silu", dict(A=NULL), -1), ("silu", dict(out=NULL), -1), ("silu", dict(s=NULL), -1),
    ("silu", dict(N=1008), -2), ("silu", dict(group=128), -3), ("silu", dict(out=ODD), -4),
    ("silu", dict(plan=w4.make_plan(w4.PATH_MFMA, 1, 4)), -8),
    ("argmax", dict(out=NULL), -1), ("argmax", dict(val=NULL), -1), ("argmax", dict(M=17), -2),
    ("argmax", dict(group=128), -3), ("argmax", dict(out=ctypes.c_void_p(0x20002)), -4),
    ("argmax", dict(wsb=65535), -5), ("argmax", dict(ws=NULL), -5),
    ("argmax", dict(plan=w4.make_plan(w4.PATH_MFMA, 1, 4, 2)), -8),
    ("f32", dict(out=NULL), -1), ("f32", dict(K=520), -2), ("f32", dict(group=128), -3),
    ("f32", dict(plan=w4.make_plan(w4.PATH_MFMA, 1, 1, 1, w4.ASRC_RING)), -8),
])
def test_nvfp4_epilogue_argument_errors(kind, kw, status):
    assert _nv_epi(kind, **kw) == status


@pytest.mark.parametrize("kind", ["silu", "argmax", "f32"])
def test_epilogue_auto_plans_have_a_kernel(kind):
    # without a device a call that passed every host check (the automatic
    # plan and its compiled kernel included) returns "no device": so no
    # automatic plan of any mode, format or row count lacks a kernel
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = w4.lib()
    shapes = ((8192, 5120), (34816, 5120), (5120, 17408), (248320, 5120), (1024, 512), (64, 128),
              (2048, 1 << 24))
    for M in range(1, 17):
        for N, K in shapes:
            assert _nv_epi(kind, M=M, N=N, K=K, wsb=1 << 40) == -6, (kind, M, N, K)
            g = dict(M=M, N=N, K=K, group=128, ws=P, wsb=1 << 40)
            if kind == "silu":
                st = L.w4a16_gemm_silu_mul(P, P, P, P2, M, N, K, 128, P, 1 << 40, NULL)
            elif kind == "argmax":
                st = L.w4a16_gemm_argmax(P, P, P, P2, P2, M, N, K, 128, P, 1 << 40, NULL)
            else:
                st = L.w4a16_gemm_f32(P, P, P, P2, M, N, K, 128, P, 1 << 40, NULL)
            assert st == -6, (kind, g)


def test_split_n_plans():
    # four wavefronts split the columns: compiled for kwaves = 4 only, any row
    # count (run-time M), both formats; the strip is kwaves x tiles tiles
    N, K = 8192, 5120
    for M in (1, 4, 5, 16):
        for t, d in ((1, 2), (1, 4), (2, 2), (2, 3), (2, 4), (4, 2)):
            assert w4.plan_ok(M, N, K, w4.make_plan(w4.PATH_MFMA, t, 4, 1, w4.ASRC_SPLITN, d)), (M, t, d)
        assert not w4.plan_ok(M, N, K, w4.make_plan(w4.PATH_MFMA, 2, 8, 1, w4.ASRC_SPLITN, 2))
        assert not w4.plan_ok(M, N, K, w4.make_plan(w4.PATH_MFMA, 2, 2, 1, w4.ASRC_SPLITN, 4))
        for t, d in ((2, 2), (2, 4), (1, 4), (4, 2)):
            assert w4.nvfp4_plan_ok(M, N, K, w4.make_plan(w4.PATH_MFMA, t, 4, 1, w4.ASRC_SPLITN, d)), (M, t, d)
    # split-K partials as for any plan: [S][M][N] fp32 after the counter region
    p = w4.make_plan(w4.PATH_MFMA, 2, 4, 4, w4.ASRC_SPLITN, 2)
    assert w4.workspace_bytes(16, N, K, p) == 65536 + 4 * 16 * N * 4
    # strips of 4 x 2 tiles: 8192 / 16 / 8 = 64 strips x 4 splits
    assert w4.plan_ok(16, N, K, p)
