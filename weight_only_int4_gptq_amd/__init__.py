"""Python binding of the gfx950 W4A16 decode/verify matmul library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libw4a16.so`` (built from ``csrc/``), called through its C ABI
(``include/w4a16.h``).  PyTorch supplies device memory and the current
stream.  If the library is not built, or a call returns an error status,
the functions raise: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

OK = 0
PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2
ASRC_LDS, ASRC_GLOBAL, ASRC_RING, ASRC_SPLITN = 0, 1, 2, 3
GROUP = 128
NVFP4_GROUP = 16


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("tiles", ctypes.c_int), ("kwaves", ctypes.c_int),
                ("splits", ctypes.c_int), ("asrc", ctypes.c_int), ("depth", ctypes.c_int),
                ("whole", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}

    def __repr__(self):
        return f"Plan({self.as_dict()})"


_lib = None


def lib():
    """The loaded libw4a16.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python weight_only_int4_gptq_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.w4a16_status_string.argtypes = [I]
        L.w4a16_status_string.restype = ctypes.c_char_p
        L.w4a16_repacked_bytes.argtypes = [I, I]
        L.w4a16_repacked_bytes.restype = S
        L.w4a16_repack_weights.argtypes = [P, P, I, I, P]
        L.w4a16_get_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_check_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_check_plan.restype = I
        L.w4a16_workspace_bytes.argtypes = [I, I, I]
        L.w4a16_workspace_bytes.restype = S
        L.w4a16_workspace_bytes_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_workspace_bytes_plan.restype = S
        L.w4a16_gemm.argtypes = [P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_plan.argtypes = [P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_gemm_silu_mul.argtypes = [P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_argmax.argtypes = [P, P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_f32.argtypes = [P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_f32_plan.argtypes = [P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_gemm_argmax_plan.argtypes = [P, P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_gemm_silu_mul_plan.argtypes = [P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_dequant_debug.argtypes = [P, P, P, I, I, P]
        L.w4a16_unpack_debug.argtypes = [P, P, I, I, P]
        F = ctypes.c_float
        L.w4a16_nvfp4_repacked_bytes.argtypes = [I, I]
        L.w4a16_nvfp4_repacked_bytes.restype = S
        L.w4a16_nvfp4_repacked_scale_bytes.argtypes = [I, I]
        L.w4a16_nvfp4_repacked_scale_bytes.restype = S
        L.w4a16_nvfp4_repack_weights.argtypes = [P, P, I, I, P]
        L.w4a16_nvfp4_repack_scales.argtypes = [P, P, I, I, P]
        L.w4a16_nvfp4_get_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_nvfp4_check_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_nvfp4_workspace_bytes.argtypes = [I, I, I]
        L.w4a16_nvfp4_workspace_bytes.restype = S
        L.w4a16_nvfp4_workspace_bytes_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_nvfp4_workspace_bytes_plan.restype = S
        L.w4a16_nvfp4_gemm.argtypes = [P, P, P, F, P, I, I, I, I, P, S, P]
        L.w4a16_nvfp4_gemm_plan.argtypes = [P, P, P, F, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_nvfp4_dequant.argtypes = [P, P, P, I, I, P]
        PL = ctypes.POINTER(Plan)
        L.w4a16_nvfp4_gemm_silu_mul.argtypes = [P, P, P, F, P, I, I, I, I, P, S, P]
        L.w4a16_nvfp4_gemm_silu_mul_plan.argtypes = [P, P, P, F, P, I, I, I, I, P, S, PL, P]
        L.w4a16_nvfp4_gemm_argmax.argtypes = [P, P, P, F, P, P, I, I, I, I, P, S, P]
        L.w4a16_nvfp4_gemm_argmax_plan.argtypes = [P, P, P, F, P, P, I, I, I, I, P, S, PL, P]
        L.w4a16_nvfp4_gemm_f32.argtypes = [P, P, P, F, P, I, I, I, I, P, S, P]
        L.w4a16_nvfp4_gemm_f32_plan.argtypes = [P, P, P, F, P, I, I, I, I, P, S, PL, P]
        for f in ("w4a16_nvfp4_repack_weights", "w4a16_nvfp4_repack_scales", "w4a16_nvfp4_get_plan",
                  "w4a16_nvfp4_check_plan", "w4a16_nvfp4_gemm", "w4a16_nvfp4_gemm_plan",
                  "w4a16_nvfp4_dequant", "w4a16_nvfp4_gemm_silu_mul", "w4a16_nvfp4_gemm_silu_mul_plan",
                  "w4a16_nvfp4_gemm_argmax", "w4a16_nvfp4_gemm_argmax_plan", "w4a16_nvfp4_gemm_f32",
                  "w4a16_nvfp4_gemm_f32_plan"):
            getattr(L, f).restype = I
        for f in ("w4a16_repack_weights", "w4a16_get_plan", "w4a16_gemm", "w4a16_gemm_plan",
                  "w4a16_gemm_silu_mul", "w4a16_gemm_silu_mul_plan", "w4a16_gemm_argmax",
                  "w4a16_gemm_argmax_plan", "w4a16_gemm_f32", "w4a16_gemm_f32_plan",
                  "w4a16_dequant_debug", "w4a16_unpack_debug"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().w4a16_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise W4A16Error(status, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# ---------------------------------------------------------------- argument checks
# Every wrapper checks its tensors before the library sees a pointer: a
# wrong shape, dtype or size would otherwise make a kernel read or write past
# an allocation.  The C ABI checks what it can see (shapes, alignment, group,
# workspace size); these checks add what only the tensors know.

_BITS16 = (torch.bfloat16, torch.int16, torch.float16) + ((torch.uint16,) if hasattr(torch, "uint16") else ())


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _require(cond: bool, what: str, msg: str):
    if not cond:
        raise ValueError(f"{what}: {msg}")


def _check_dense(t: torch.Tensor, name: str, what: str):
    _require(isinstance(t, torch.Tensor), what, f"{name} must be a torch.Tensor")
    _require(t.is_contiguous(), what, f"{name} must be contiguous")


def _check_device(what: str, *ts):
    devs = {t.device for t in ts if t is not None}
    _require(all(d.type == "cuda" for d in devs), what, "tensors must be on a CUDA (HIP) device")
    _require(len(devs) == 1, what, f"tensors must be on one device, got {sorted(map(str, devs))}")


def _check_a(A: torch.Tensor, what: str):
    _check_dense(A, "A", what)
    _require(A.dim() == 2, what, f"A must be 2-D [M, K], got shape {tuple(A.shape)}")
    _require(A.dtype == torch.bfloat16, what, f"A must be bfloat16, got {A.dtype}")
    M, K = A.shape
    _require(1 <= M <= 16, what, f"A must have 1..16 rows, got {M}")
    _require(K > 0 and K % GROUP == 0, what, f"K must be a positive multiple of {GROUP}, got {K}")
    return M, K


def _check_weights(blob, scales, K, N, what, nvfp4=False):
    _check_dense(blob, "blob", what)
    _check_dense(scales, "scales", what)
    _require(N > 0 and N % 16 == 0, what, f"N must be a positive multiple of 16, got {N}")
    _require(_nbytes(blob) >= K * N // 2, what,
             f"blob holds {_nbytes(blob)} bytes, a {K} x {N} matrix needs {K * N // 2}")
    if nvfp4:
        need = K * N // NVFP4_GROUP
        _require(_nbytes(scales) >= need, what, f"scales hold {_nbytes(scales)} bytes, need {need}")
    else:
        _require(scales.dtype in _BITS16, what, f"scales must be bf16 (16-bit), got {scales.dtype}")
        _require(scales.numel() == (K // GROUP) * N, what,
                 f"scales must be [K/128, N] = [{K // GROUP}, {N}], got {tuple(scales.shape)}")
        if scales.dim() == 2:
            _require(tuple(scales.shape) == (K // GROUP, N), what,
                     f"scales must be [K/128, N] = [{K // GROUP}, {N}], got {tuple(scales.shape)}")


def _out(out, shape, dtype, like, what):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _check_dense(out, "out", what)
    _require(out.dtype == dtype, what, f"out must be {dtype}, got {out.dtype}")
    _require(tuple(out.shape) == tuple(shape), what, f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    return out


def _check_plan(plan, what):
    _require(plan is None or isinstance(plan, Plan), what, "plan must be a Plan or None")


def _workspace(A, need, workspace, what):
    """The caller's workspace (checked), or the shared zero-filled one of A's device."""
    if workspace is None:
        return _shared_workspace(A.device, need) if need else None
    _check_dense(workspace, "workspace", what)
    _require(_nbytes(workspace) >= need, what, f"workspace holds {_nbytes(workspace)} bytes, need {need}")
    return workspace


# ---------------------------------------------------------------- GPTQ INT4

def repacked_bytes(K: int, N: int) -> int:
    return int(lib().w4a16_repacked_bytes(K, N))


def repack_weights(qweight: torch.Tensor, K: int, N: int, out: torch.Tensor | None = None):
    """GPTQ words (int32/uint32 device tensor [K/8, N]) -> repacked blob (uint8 [K*N/2]).

    The one-time preparation of a checkpoint matrix; its bf16 scales [K/128, N]
    are passed to the matmul as they are.
    """
    what = "w4a16_repack_weights"
    _check_dense(qweight, "qweight", what)
    _require(qweight.element_size() == 4, what, f"qweight must hold 32-bit words, got {qweight.dtype}")
    _require(K > 0 and K % GROUP == 0 and N > 0 and N % 16 == 0, what, f"invalid shape K={K}, N={N}")
    _require(qweight.numel() == (K // 8) * N, what, f"qweight must be [K/8, N] = [{K // 8}, {N}], got {tuple(qweight.shape)}")
    nbytes = repacked_bytes(K, N)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    _check_dense(out, "out", what)
    _require(_nbytes(out) >= nbytes, what, f"out holds {_nbytes(out)} bytes, need {nbytes}")
    _check_device(what, qweight, out)
    _check(lib().w4a16_repack_weights(_ptr(qweight), _ptr(out), K, N, _stream(qweight)), what)
    return out


def get_plan(M: int, N: int, K: int) -> Plan:
    p = Plan()
    _check(lib().w4a16_get_plan(M, N, K, ctypes.byref(p)), "w4a16_get_plan")
    return p


def make_plan(path: int, tiles: int, kwaves: int, splits: int = 1, asrc: int = ASRC_LDS,
              depth: int = 0, whole: int = 0) -> Plan:
    return Plan(path, tiles, kwaves, splits, asrc, depth, whole)


def plan_ok(M: int, N: int, K: int, plan: Plan) -> bool:
    """True if the library has a kernel for `plan` at (M, N, K) and its LDS fits."""
    return lib().w4a16_check_plan(M, N, K, ctypes.byref(plan)) == OK


def workspace_bytes(M: int, N: int, K: int, plan: Plan | None = None) -> int:
    """Workspace bytes for `plan` at (M, N, K); with plan=None, bytes that serve
    every call kind at this shape with its automatic plan."""
    if plan is None:
        return int(lib().w4a16_workspace_bytes(M, N, K))
    return int(lib().w4a16_workspace_bytes_plan(M, N, K, ctypes.byref(plan)))


_workspaces: dict = {}


def _shared_workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-filled split-K workspace per device, grown on demand.

    Every call leaves its counters at zero again, so one buffer serves all
    calls issued in order on one stream; calls that run concurrently need
    their own (pass ``workspace=``).
    """
    key = str(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _run(entry, entry_plan, what, A, blob, scales, N, out, plan, workspace, group, extra_out=()):
    """Shared marshalling of the matmul calls: out-arguments, workspace, stream."""
    M, K = A.shape
    _check_device(what, A, blob, scales, out, workspace, *extra_out)
    need = workspace_bytes(M, N, K, plan)
    ws = _workspace(A, need, workspace, what)
    outs = [_ptr(o) for o in ((out,) if out is not None else extra_out)]
    ws_bytes = _nbytes(ws) if ws is not None else 0
    if plan is None:
        st = entry(_ptr(A), _ptr(blob), _ptr(scales), *outs, M, N, K, group, _ptr(ws), ws_bytes, _stream(A))
    else:
        st = entry_plan(_ptr(A), _ptr(blob), _ptr(scales), *outs, M, N, K, group, _ptr(ws), ws_bytes,
                        ctypes.byref(plan), _stream(A))
    _check(st, what)


def gemm(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
         out: torch.Tensor | None = None, plan: Plan | None = None,
         workspace: torch.Tensor | None = None, group: int = GROUP):
    """C[M, N] = A[M, K] . dequant(blob, scales); A and C bf16 device tensors.

    ``blob`` comes from ``repack_weights``; ``scales`` are the checkpoint's bf16 [K/128, N].
    """
    what = "w4a16_gemm"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what)
    _check_plan(plan, what)
    out = _out(out, (M, N), torch.bfloat16, A, what)
    _run(lib().w4a16_gemm, lib().w4a16_gemm_plan, what, A, blob, scales, N, out, plan, workspace, group)
    return out


def gemm_silu_mul(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
                  out: torch.Tensor | None = None, plan: Plan | None = None,
                  workspace: torch.Tensor | None = None, group: int = GROUP):
    """H[M, N/2] = silu(C[:, :N/2]) * C[:, N/2:] with C = A . dequant(fused gate/up weight [K, N])."""
    what = "w4a16_gemm_silu_mul"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what)
    _require(N % 32 == 0, what, f"the fused width N must be a multiple of 32, got {N}")
    _check_plan(plan, what)
    out = _out(out, (M, N // 2), torch.bfloat16, A, what)
    _run(lib().w4a16_gemm_silu_mul, lib().w4a16_gemm_silu_mul_plan, what, A, blob, scales, N, out, plan,
         workspace, group)
    return out


def gemm_f32(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
             out: torch.Tensor | None = None, plan: Plan | None = None,
             workspace: torch.Tensor | None = None, group: int = GROUP):
    """C[M, N] = A . dequant(blob, scales) as unrounded fp32 (a K shard's partial sum)."""
    what = "w4a16_gemm_f32"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what)
    _check_plan(plan, what)
    out = _out(out, (M, N), torch.float32, A, what)
    _run(lib().w4a16_gemm_f32, lib().w4a16_gemm_f32_plan, what, A, blob, scales, N, out, plan, workspace, group)
    return out


ARGMAX_WORKSPACE_BYTES = 65536   # the workspace's counter region


def gemm_argmax(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
                plan: Plan | None = None, workspace: torch.Tensor | None = None, group: int = GROUP):
    """Per-row argmax of C = A . dequant(W) (lowest column among equal values).

    Returns (idx int32 [M], val float32 [M]) device tensors.
    """
    what = "w4a16_gemm_argmax"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what)
    _check_plan(plan, what)
    idx = torch.empty(M, dtype=torch.int32, device=A.device)
    val = torch.empty(M, dtype=torch.float32, device=A.device)
    _check_device(what, A, blob, scales, workspace)
    ws = _workspace(A, ARGMAX_WORKSPACE_BYTES, workspace, what)
    if plan is None:
        st = lib().w4a16_gemm_argmax(_ptr(A), _ptr(blob), _ptr(scales), _ptr(idx), _ptr(val), M, N, K,
                                     group, _ptr(ws), _nbytes(ws), _stream(A))
    else:
        st = lib().w4a16_gemm_argmax_plan(_ptr(A), _ptr(blob), _ptr(scales), _ptr(idx), _ptr(val), M, N,
                                          K, group, _ptr(ws), _nbytes(ws), ctypes.byref(plan), _stream(A))
    _check(st, what)
    return idx, val


def dequant_debug(blob: torch.Tensor, scales: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Test export: fp32 W[K, N] = (q - 8) * s from the device dequantization."""
    what = "w4a16_dequant_debug"
    _check_weights(blob, scales, K, N, what)
    W = torch.empty((K, N), dtype=torch.float32, device=blob.device)
    _check_device(what, blob, scales, W)
    _check(lib().w4a16_dequant_debug(_ptr(blob), _ptr(scales), _ptr(W), K, N, _stream(blob)), what)
    return W


def unpack_debug(blob: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Test export: codes uint8 [K, N] from the device unpacking."""
    what = "w4a16_unpack_debug"
    _check_dense(blob, "blob", what)
    _require(_nbytes(blob) >= K * N // 2, what, f"blob holds {_nbytes(blob)} bytes, need {K * N // 2}")
    codes = torch.empty((K, N), dtype=torch.uint8, device=blob.device)
    _check_device(what, blob, codes)
    _check(lib().w4a16_unpack_debug(_ptr(blob), _ptr(codes), K, N, _stream(blob)), what)
    return codes


# ---------------------------------------------------------------- NVFP4

def nvfp4_repacked_bytes(K: int, N: int) -> int:
    return int(lib().w4a16_nvfp4_repacked_bytes(K, N))


def nvfp4_repacked_scale_bytes(K: int, N: int) -> int:
    return int(lib().w4a16_nvfp4_repacked_scale_bytes(K, N))


def nvfp4_repack(packed: torch.Tensor, scales: torch.Tensor, K: int, N: int):
    """One-time repacks of NVFP4 weights: packed E2M1 codes (uint8 device
    tensor [N, K/2]) and E4M3 block scales (uint8 [N, K/16]) ->
    (blob uint8 [K*N/2], repacked scales uint8 [K*N/16])."""
    what = "w4a16_nvfp4_repack"
    _check_dense(packed, "packed", what)
    _check_dense(scales, "scales", what)
    _require(K > 0 and K % GROUP == 0 and N > 0 and N % 16 == 0, what, f"invalid shape K={K}, N={N}")
    _require(packed.dtype == torch.uint8 and packed.numel() == N * (K // 2), what,
             f"packed must be uint8 [N, K/2] = [{N}, {K // 2}], got {packed.dtype} {tuple(packed.shape)}")
    _require(scales.dtype == torch.uint8 and scales.numel() == N * (K // NVFP4_GROUP), what,
             f"scales must be uint8 [N, K/16] = [{N}, {K // NVFP4_GROUP}], got {scales.dtype} {tuple(scales.shape)}")
    _check_device(what, packed, scales)
    blob = torch.empty(max(nvfp4_repacked_bytes(K, N), 1), dtype=torch.uint8, device=packed.device)
    sc = torch.empty(max(nvfp4_repacked_scale_bytes(K, N), 1), dtype=torch.uint8, device=packed.device)
    _check(lib().w4a16_nvfp4_repack_weights(_ptr(packed), _ptr(blob), K, N, _stream(packed)),
           "w4a16_nvfp4_repack_weights")
    _check(lib().w4a16_nvfp4_repack_scales(_ptr(scales), _ptr(sc), K, N, _stream(scales)),
           "w4a16_nvfp4_repack_scales")
    return blob, sc


def nvfp4_get_plan(M: int, N: int, K: int) -> Plan:
    p = Plan()
    _check(lib().w4a16_nvfp4_get_plan(M, N, K, ctypes.byref(p)), "w4a16_nvfp4_get_plan")
    return p


def nvfp4_plan_ok(M: int, N: int, K: int, plan: Plan) -> bool:
    return lib().w4a16_nvfp4_check_plan(M, N, K, ctypes.byref(plan)) == OK


def nvfp4_workspace_bytes(M: int, N: int, K: int, plan: Plan | None = None) -> int:
    if plan is None:
        return int(lib().w4a16_nvfp4_workspace_bytes(M, N, K))
    return int(lib().w4a16_nvfp4_workspace_bytes_plan(M, N, K, ctypes.byref(plan)))


def _run_nv(entry, entry_plan, what, A, blob, scales, alpha, N, outs, plan, workspace, group, need=None):
    M, K = A.shape
    _check_device(what, A, blob, scales, workspace, *outs)
    if need is None:
        need = nvfp4_workspace_bytes(M, N, K, plan)
    ws = _workspace(A, need, workspace, what)
    ws_bytes = _nbytes(ws) if ws is not None else 0
    ptrs = [_ptr(o) for o in outs]
    if plan is None:
        st = entry(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), *ptrs, M, N, K, group, _ptr(ws), ws_bytes,
                   _stream(A))
    else:
        st = entry_plan(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), *ptrs, M, N, K, group, _ptr(ws),
                        ws_bytes, ctypes.byref(plan), _stream(A))
    _check(st, what)


def nvfp4_gemm(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
               out: torch.Tensor | None = None, plan: Plan | None = None,
               workspace: torch.Tensor | None = None, group: int = NVFP4_GROUP):
    """C[M, N] = alpha * A . dequant(blob, scales) for NVFP4 weights (from ``nvfp4_repack``)."""
    what = "w4a16_nvfp4_gemm"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what, nvfp4=True)
    _check_plan(plan, what)
    out = _out(out, (M, N), torch.bfloat16, A, what)
    _run_nv(lib().w4a16_nvfp4_gemm, lib().w4a16_nvfp4_gemm_plan, what, A, blob, scales, alpha, N, (out,), plan,
            workspace, group)
    return out


def nvfp4_gemm_silu_mul(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
                        out: torch.Tensor | None = None, plan: Plan | None = None,
                        workspace: torch.Tensor | None = None, group: int = NVFP4_GROUP):
    """H[M, N/2] = silu(C[:, :N/2]) * C[:, N/2:], C = alpha * A . dequant(NVFP4 gate/up weight [K, N])."""
    what = "w4a16_nvfp4_gemm_silu_mul"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what, nvfp4=True)
    _require(N % 32 == 0, what, f"the fused width N must be a multiple of 32, got {N}")
    _check_plan(plan, what)
    out = _out(out, (M, N // 2), torch.bfloat16, A, what)
    _run_nv(lib().w4a16_nvfp4_gemm_silu_mul, lib().w4a16_nvfp4_gemm_silu_mul_plan, what, A, blob, scales, alpha,
            N, (out,), plan, workspace, group)
    return out


def nvfp4_gemm_argmax(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
                      plan: Plan | None = None, workspace: torch.Tensor | None = None,
                      group: int = NVFP4_GROUP):
    """Per-row argmax of C = alpha * A . dequant(NVFP4 W): (idx int32 [M], val float32 [M])."""
    what = "w4a16_nvfp4_gemm_argmax"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what, nvfp4=True)
    _check_plan(plan, what)
    idx = torch.empty(M, dtype=torch.int32, device=A.device)
    val = torch.empty(M, dtype=torch.float32, device=A.device)
    _run_nv(lib().w4a16_nvfp4_gemm_argmax, lib().w4a16_nvfp4_gemm_argmax_plan, what, A, blob, scales, alpha, N,
            (idx, val), plan, workspace, group, need=ARGMAX_WORKSPACE_BYTES)
    return idx, val


def nvfp4_gemm_f32(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
                   out: torch.Tensor | None = None, plan: Plan | None = None,
                   workspace: torch.Tensor | None = None, group: int = NVFP4_GROUP):
    """C = alpha * A . dequant(NVFP4 W) as unrounded fp32 (a K shard's partial sum)."""
    what = "w4a16_nvfp4_gemm_f32"
    M, K = _check_a(A, what)
    _check_weights(blob, scales, K, N, what, nvfp4=True)
    _check_plan(plan, what)
    out = _out(out, (M, N), torch.float32, A, what)
    _run_nv(lib().w4a16_nvfp4_gemm_f32, lib().w4a16_nvfp4_gemm_f32_plan, what, A, blob, scales, alpha, N, (out,),
            plan, workspace, group)
    return out


def nvfp4_dequant(blob: torch.Tensor, scales: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Test export: fp32 W[K, N] = e2m1 * e4m3 from the device conversions (repacked inputs)."""
    what = "w4a16_nvfp4_dequant"
    _check_weights(blob, scales, K, N, what, nvfp4=True)
    W = torch.empty((K, N), dtype=torch.float32, device=blob.device)
    _check_device(what, blob, scales, W)
    _check(lib().w4a16_nvfp4_dequant(_ptr(blob), _ptr(scales), _ptr(W), K, N, _stream(blob)), what)
    return W
