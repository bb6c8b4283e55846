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
                ("splits", ctypes.c_int), ("asrc", ctypes.c_int), ("depth", ctypes.c_int)]

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
        L.w4a16_repacked_scale_bytes.argtypes = [I, I]
        L.w4a16_repacked_scale_bytes.restype = S
        L.w4a16_repack_scales.argtypes = [P, P, I, I, P]
        L.w4a16_repack_scales.restype = I
        L.w4a16_get_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_check_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_check_plan.restype = I
        L.w4a16_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_workspace_bytes.restype = S
        L.w4a16_gemm.argtypes = [P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_plan.argtypes = [P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_gemm_silu_mul.argtypes = [P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_argmax.argtypes = [P, P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_f32.argtypes = [P, P, P, P, I, I, I, I, P, S, P]
        L.w4a16_gemm_f32_plan.argtypes = [P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_gemm_argmax_plan.argtypes = [P, P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_gemm_silu_mul_plan.argtypes = [P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(Plan), P]
        L.w4a16_dequant.argtypes = [P, P, P, I, I, P]
        L.w4a16_unpack.argtypes = [P, P, I, I, P]
        F = ctypes.c_float
        L.w4a16_nvfp4_repacked_bytes.argtypes = [I, I]
        L.w4a16_nvfp4_repacked_bytes.restype = S
        L.w4a16_nvfp4_repacked_scale_bytes.argtypes = [I, I]
        L.w4a16_nvfp4_repacked_scale_bytes.restype = S
        L.w4a16_nvfp4_repack_weights.argtypes = [P, P, I, I, P]
        L.w4a16_nvfp4_repack_scales.argtypes = [P, P, I, I, P]
        L.w4a16_nvfp4_get_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_nvfp4_check_plan.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_nvfp4_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(Plan)]
        L.w4a16_nvfp4_workspace_bytes.restype = S
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
                  "w4a16_dequant", "w4a16_unpack"):
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


def repacked_bytes(K: int, N: int) -> int:
    return int(lib().w4a16_repacked_bytes(K, N))


def repack_weights(qweight: torch.Tensor, K: int, N: int, out: torch.Tensor | None = None):
    """GPTQ words (int32/uint32 device tensor [K/8, N]) -> repacked blob (uint8 [K*N/2])."""
    nbytes = repacked_bytes(K, N)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    _check(lib().w4a16_repack_weights(_ptr(qweight), _ptr(out), K, N, _stream(qweight)),
           "w4a16_repack_weights")
    return out


def repack_scales(scales: torch.Tensor, K: int, N: int, out: torch.Tensor | None = None):
    """bf16 scales (16-bit device tensor [K/128, N]) -> tile-order scales (int16 [K/128 * N])."""
    if out is None:
        out = torch.empty(max((K // GROUP) * N, 1), dtype=torch.int16, device=scales.device)
    _check(lib().w4a16_repack_scales(_ptr(scales), _ptr(out), K, N, _stream(scales)),
           "w4a16_repack_scales")
    return out


def repack(qweight: torch.Tensor, scales: torch.Tensor, K: int, N: int):
    """Both one-time repacks: (blob, repacked scales)."""
    return repack_weights(qweight, K, N), repack_scales(scales, K, N)


def get_plan(M: int, N: int, K: int) -> Plan:
    p = Plan()
    _check(lib().w4a16_get_plan(M, N, K, ctypes.byref(p)), "w4a16_get_plan")
    return p


def make_plan(path: int, tiles: int, kwaves: int, splits: int = 1, asrc: int = ASRC_LDS,
              depth: int = 0) -> Plan:
    return Plan(path, tiles, kwaves, splits, asrc, depth)


def plan_ok(M: int, N: int, K: int, plan: Plan) -> bool:
    """True if the library has a kernel for `plan` at (M, N, K) and its LDS fits."""
    return lib().w4a16_check_plan(M, N, K, ctypes.byref(plan)) == OK


def workspace_bytes(M: int, N: int, K: int, plan: Plan | None = None) -> int:
    return int(lib().w4a16_workspace_bytes(M, N, K, ctypes.byref(plan) if plan else None))


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


def gemm(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
         out: torch.Tensor | None = None, plan: Plan | None = None,
         workspace: torch.Tensor | None = None, group: int = GROUP):
    """C[M, N] = A[M, K] . dequant(blob, scales); A and C bf16 device tensors.

    ``blob`` and ``scales`` come from ``repack`` (weights and scales repacked once).
    """
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if workspace is None:
        need = workspace_bytes(M, N, K, plan)
        if need:
            workspace = _shared_workspace(A.device, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if plan is None:
        st = lib().w4a16_gemm(_ptr(A), _ptr(blob), _ptr(scales), _ptr(out), M, N, K, group,
                              _ptr(workspace), ws_bytes, _stream(A))
    else:
        st = lib().w4a16_gemm_plan(_ptr(A), _ptr(blob), _ptr(scales), _ptr(out), M, N, K, group,
                                   _ptr(workspace), ws_bytes, ctypes.byref(plan), _stream(A))
    _check(st, "w4a16_gemm")
    return out


def gemm_silu_mul(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
                  out: torch.Tensor | None = None, plan: Plan | None = None,
                  workspace: torch.Tensor | None = None, group: int = GROUP):
    """H[M, N/2] = silu(C[:, :N/2]) * C[:, N/2:] with C = A . dequant(fused gate/up weight [K, N])."""
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=A.device)
    if workspace is None:
        need = workspace_bytes(M, N, K, plan)
        if need:
            workspace = _shared_workspace(A.device, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if plan is None:
        st = lib().w4a16_gemm_silu_mul(_ptr(A), _ptr(blob), _ptr(scales), _ptr(out), M, N, K, group,
                                       _ptr(workspace), ws_bytes, _stream(A))
    else:
        st = lib().w4a16_gemm_silu_mul_plan(_ptr(A), _ptr(blob), _ptr(scales), _ptr(out), M, N, K, group,
                                            _ptr(workspace), ws_bytes, ctypes.byref(plan), _stream(A))
    _check(st, "w4a16_gemm_silu_mul")
    return out


def gemm_f32(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
             out: torch.Tensor | None = None, plan: Plan | None = None,
             workspace: torch.Tensor | None = None, group: int = GROUP):
    """C[M, N] = A . dequant(blob, scales) as unrounded fp32 (a K shard's partial sum)."""
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if workspace is None:
        need = workspace_bytes(M, N, K, plan)
        if need:
            workspace = _shared_workspace(A.device, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if plan is None:
        st = lib().w4a16_gemm_f32(_ptr(A), _ptr(blob), _ptr(scales), _ptr(out), M, N, K, group,
                                  _ptr(workspace), ws_bytes, _stream(A))
    else:
        st = lib().w4a16_gemm_f32_plan(_ptr(A), _ptr(blob), _ptr(scales), _ptr(out), M, N, K, group,
                                       _ptr(workspace), ws_bytes, ctypes.byref(plan), _stream(A))
    _check(st, "w4a16_gemm_f32")
    return out


ARGMAX_WORKSPACE_BYTES = 65536   # the workspace's counter region


def gemm_argmax(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, N: int,
                plan: Plan | None = None, workspace: torch.Tensor | None = None, group: int = GROUP):
    """Per-row argmax of C = A . dequant(W) (lowest column among equal values).

    Returns (idx int32 [M], val float32 [M]) device tensors.
    """
    M, K = A.shape
    idx = torch.empty(M, dtype=torch.int32, device=A.device)
    val = torch.empty(M, dtype=torch.float32, device=A.device)
    if workspace is None:
        workspace = _shared_workspace(A.device, ARGMAX_WORKSPACE_BYTES)
    ws_bytes = workspace.numel() * workspace.element_size()
    if plan is None:
        st = lib().w4a16_gemm_argmax(_ptr(A), _ptr(blob), _ptr(scales), _ptr(idx), _ptr(val), M, N, K,
                                     group, _ptr(workspace), ws_bytes, _stream(A))
    else:
        st = lib().w4a16_gemm_argmax_plan(_ptr(A), _ptr(blob), _ptr(scales), _ptr(idx), _ptr(val), M, N,
                                          K, group, _ptr(workspace), ws_bytes, ctypes.byref(plan),
                                          _stream(A))
    _check(st, "w4a16_gemm_argmax")
    return idx, val


def dequant(blob: torch.Tensor, scales: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Test export: fp32 W[K, N] = (q - 8) * s from the device dequantization (repacked scales)."""
    W = torch.empty((K, N), dtype=torch.float32, device=blob.device)
    _check(lib().w4a16_dequant(_ptr(blob), _ptr(scales), _ptr(W), K, N, _stream(blob)),
           "w4a16_dequant")
    return W


def unpack(blob: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Test export: codes uint8 [K, N] from the device unpacking."""
    codes = torch.empty((K, N), dtype=torch.uint8, device=blob.device)
    _check(lib().w4a16_unpack(_ptr(blob), _ptr(codes), K, N, _stream(blob)), "w4a16_unpack")
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
    return int(lib().w4a16_nvfp4_workspace_bytes(M, N, K, ctypes.byref(plan) if plan else None))


def nvfp4_gemm(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
               out: torch.Tensor | None = None, plan: Plan | None = None,
               workspace: torch.Tensor | None = None, group: int = NVFP4_GROUP):
    """C[M, N] = alpha * A . dequant(blob, scales) for NVFP4 weights (from ``nvfp4_repack``)."""
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if workspace is None:
        need = nvfp4_workspace_bytes(M, N, K, plan)
        if need:
            workspace = _shared_workspace(A.device, need)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if plan is None:
        st = lib().w4a16_nvfp4_gemm(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(out), M, N, K,
                                    group, _ptr(workspace), ws_bytes, _stream(A))
    else:
        st = lib().w4a16_nvfp4_gemm_plan(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(out), M, N,
                                         K, group, _ptr(workspace), ws_bytes, ctypes.byref(plan),
                                         _stream(A))
    _check(st, "w4a16_nvfp4_gemm")
    return out


def _nv_ws(A, N, K, plan, workspace, minimum=0):
    M = A.shape[0]
    if workspace is None:
        need = max(nvfp4_workspace_bytes(M, N, K, plan), minimum)
        if need:
            workspace = _shared_workspace(A.device, need)
    return workspace, (workspace.numel() * workspace.element_size() if workspace is not None else 0)


def nvfp4_gemm_silu_mul(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
                        out: torch.Tensor | None = None, plan: Plan | None = None,
                        workspace: torch.Tensor | None = None, group: int = NVFP4_GROUP):
    """H[M, N/2] = silu(C[:, :N/2]) * C[:, N/2:], C = alpha * A . dequant(NVFP4 gate/up weight [K, N])."""
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=A.device)
    ws, wsb = _nv_ws(A, N, K, plan, workspace)
    if plan is None:
        st = lib().w4a16_nvfp4_gemm_silu_mul(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(out), M, N, K,
                                             group, _ptr(ws), wsb, _stream(A))
    else:
        st = lib().w4a16_nvfp4_gemm_silu_mul_plan(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(out), M,
                                                  N, K, group, _ptr(ws), wsb, ctypes.byref(plan), _stream(A))
    _check(st, "w4a16_nvfp4_gemm_silu_mul")
    return out


def nvfp4_gemm_argmax(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
                      plan: Plan | None = None, workspace: torch.Tensor | None = None,
                      group: int = NVFP4_GROUP):
    """Per-row argmax of C = alpha * A . dequant(NVFP4 W): (idx int32 [M], val float32 [M])."""
    M, K = A.shape
    idx = torch.empty(M, dtype=torch.int32, device=A.device)
    val = torch.empty(M, dtype=torch.float32, device=A.device)
    if workspace is None:
        workspace = _shared_workspace(A.device, ARGMAX_WORKSPACE_BYTES)
    wsb = workspace.numel() * workspace.element_size()
    if plan is None:
        st = lib().w4a16_nvfp4_gemm_argmax(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(idx), _ptr(val),
                                           M, N, K, group, _ptr(workspace), wsb, _stream(A))
    else:
        st = lib().w4a16_nvfp4_gemm_argmax_plan(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(idx),
                                                _ptr(val), M, N, K, group, _ptr(workspace), wsb,
                                                ctypes.byref(plan), _stream(A))
    _check(st, "w4a16_nvfp4_gemm_argmax")
    return idx, val


def nvfp4_gemm_f32(A: torch.Tensor, blob: torch.Tensor, scales: torch.Tensor, alpha: float, N: int,
                   out: torch.Tensor | None = None, plan: Plan | None = None,
                   workspace: torch.Tensor | None = None, group: int = NVFP4_GROUP):
    """C = alpha * A . dequant(NVFP4 W) as unrounded fp32 (a K shard's partial sum)."""
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    ws, wsb = _nv_ws(A, N, K, plan, workspace)
    if plan is None:
        st = lib().w4a16_nvfp4_gemm_f32(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(out), M, N, K,
                                        group, _ptr(ws), wsb, _stream(A))
    else:
        st = lib().w4a16_nvfp4_gemm_f32_plan(_ptr(A), _ptr(blob), _ptr(scales), float(alpha), _ptr(out), M, N,
                                             K, group, _ptr(ws), wsb, ctypes.byref(plan), _stream(A))
    _check(st, "w4a16_nvfp4_gemm_f32")
    return out


def nvfp4_dequant(blob: torch.Tensor, scales: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Test export: fp32 W[K, N] = e2m1 * e4m3 from the device conversions (repacked inputs)."""
    W = torch.empty((K, N), dtype=torch.float32, device=blob.device)
    _check(lib().w4a16_nvfp4_dequant(_ptr(blob), _ptr(scales), _ptr(W), K, N, _stream(blob)),
           "w4a16_nvfp4_dequant")
    return W
