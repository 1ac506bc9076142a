"""MI355X (gfx950) W4A16 group-quantised linear layer.

A thin Python binding over the C ABI of ``libawq_mi355x.so`` (declared in
``include/awq.h``): it checks tensor dtypes, devices and shapes, passes raw
device pointers and the current HIP stream, and turns status codes into
exceptions. Every step of the computation runs in the library's HIP kernels;
PyTorch only provides device memory and streams. If the library has not been
built, every call raises ``AWQLibraryMissing``.

Functions keep the C names without the ``awq_`` prefix: ``pack``, ``unpack``,
``pack_zeros``, ``dequant``, ``linear`` (and ``linear_plan``,
``linear_workspace_bytes``, ``qweight_words``).
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

AWQ_OK = 0


class AWQLibraryMissing(RuntimeError):
    pass


class AWQError(RuntimeError):
    def __init__(self, status: int, message: str, hip_error: int = 0):
        super().__init__(f"{message} (status {status}, hip error {hip_error})")
        self.status = status
        self.hip_error = hip_error


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_k", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("tpw", ctypes.c_int32), ("x_stage", ctypes.c_int32), ("tile", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("q_heads", ctypes.c_int64), ("kv_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("capacity", ctypes.c_int64), ("max_cached", ctypes.c_int64),
                ("qkv_stride", ctypes.c_int64), ("rope_style", ctypes.c_int32), ("steps", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("softmax_scale", ctypes.c_float)]


ROPE_STYLES = {"none": 0, "half": 1, "interleaved": 2}

_lib = None
_lock = threading.Lock()

_SIGS = {
    "awq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_last_hip_error": (ctypes.c_int, []),
    "awq_abi_version": (ctypes.c_int, []),
    "awq_qweight_words": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "awq_pack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "awq_unpack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "awq_pack_zeros": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p]),
    "awq_dequant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "awq_linear_plan": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                       ctypes.POINTER(Plan)]),
    "awq_linear_workspace_bytes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "awq_linear_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    "awq_linear_workspace_bytes_ex": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                     ctypes.POINTER(Plan), ctypes.POINTER(ctypes.c_size_t)]),
    "awq_linear": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "awq_linear_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Plan), ctypes.c_void_p]),
    "awq_linear_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.POINTER(Plan), ctypes.c_void_p]),
    "awq_linear_timed": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Plan),
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "awq_linear_silu_mul": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "awq_linear_silu_mul_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.POINTER(Plan), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "awq_linear_silu_mul_plan": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                ctypes.POINTER(Plan)]),
    "awq_linear_silu_mul_workspace_bytes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int, ctypes.POINTER(Plan),
                                                           ctypes.POINTER(ctypes.c_size_t)]),
    "awq_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "awq_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    "awq_quantize_act_fp8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]),
    "awq_linear_w4a8_workspace_bytes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                       ctypes.POINTER(Plan), ctypes.POINTER(ctypes.c_size_t)]),
    "awq_linear_w4a8_plan": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                            ctypes.POINTER(Plan)]),
    "awq_linear_w4a8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "awq_linear_w4a8_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Plan),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "awq_attention_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "awq_attention_plan": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32)]),
    "awq_attention_decode": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "awq_attention_decode_timed": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p]),
}


def library():
    """Load ``libawq_mi355x.so`` (once). Raises AWQLibraryMissing if absent."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise AWQLibraryMissing(
                    f"{LIB_PATH} is not built; run `python -m weight_only_bit_awq_amd.build`")
            # Load PyTorch first so that the library binds to the HIP runtime
            # PyTorch uses (same soname): one runtime per process, so device
            # pointers and streams from torch are valid in the library.
            import torch  # noqa: F401
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _check(status: int):
    if status != AWQ_OK:
        lib = library()
        raise AWQError(status, lib.awq_status_string(status).decode(), lib.awq_last_hip_error())


def _torch():
    import torch
    return torch


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _plan(plan):
    if plan is None:
        return None
    if isinstance(plan, Plan):
        return plan
    p = Plan()
    p.path = int(plan.get("path", 0))
    p.split_k = int(plan.get("split_k", 0))
    p.waves = int(plan.get("waves", 0))
    p.tpw = int(plan.get("tpw", 0))
    p.x_stage = int(plan.get("x_stage", 0))
    p.tile = int(plan.get("tile", 0))
    return p


def abi_version() -> int:
    return library().awq_abi_version()


def qweight_words(K: int, N: int) -> int:
    return int(library().awq_qweight_words(K, N))


def pack(q):
    """q uint8 [K, N] (GPU) -> device-layout qweight (int32 tensor of bit patterns)."""
    torch = _torch()
    _need(q, torch.uint8, "q", 2)
    K, N = q.shape
    out = torch.empty(max(qweight_words(K, N), 1), dtype=torch.int32, device=q.device)
    _check(library().awq_pack(q.data_ptr(), K, N, out.data_ptr(), _stream(q.device)))
    return out


def unpack(qweight, K: int, N: int):
    torch = _torch()
    _need(qweight, torch.int32, "qweight")
    out = torch.empty((K, N), dtype=torch.uint8, device=qweight.device)
    _check(library().awq_unpack(qweight.data_ptr(), K, N, out.data_ptr(), _stream(qweight.device)))
    return out


def pack_zeros(z):
    """z uint8 [K/G, N] -> packed zero points int32 [K/G, N/8]."""
    torch = _torch()
    _need(z, torch.uint8, "z", 2)
    groups, N = z.shape
    out = torch.empty((groups, N // 8), dtype=torch.int32, device=z.device)
    _check(library().awq_pack_zeros(z.data_ptr(), groups, N, out.data_ptr(), _stream(z.device)))
    return out


def dequant(qweight, scales, zeros, K: int, N: int, group: int = 128):
    """Device qweight + fp16 scales [K/G, N] + packed zeros -> fp16 W [K, N]."""
    torch = _torch()
    _need(qweight, torch.int32, "qweight")
    _need(scales, torch.float16, "scales", 2)
    _need(zeros, torch.int32, "zeros", 2)
    out = torch.empty((K, N), dtype=torch.float16, device=qweight.device)
    _check(library().awq_dequant(qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), K, N, group,
                                 out.data_ptr(), _stream(qweight.device)))
    return out


def quantize(w, group: int = 128):
    """fp16 w [K, N] -> (qweight device words, scales fp16 [K/G, N], zeros
    int32 [K/G, N/8]): the round-to-nearest group quantiser."""
    torch = _torch()
    _need(w, torch.float16, "w", 2)
    K, N = w.shape
    if group <= 0:
        raise ValueError("group must be positive")
    # shapes the library rejects (K % group, N % 8) fail in the call below
    qw = torch.empty(qweight_words(K, N), dtype=torch.int32, device=w.device)
    scales = torch.empty((K // group, N), dtype=torch.float16, device=w.device)
    zeros = torch.empty((K // group, N // 8), dtype=torch.int32, device=w.device)
    _check(library().awq_quantize(w.data_ptr(), K, N, group, qw.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                  _stream(w.device)))
    return qw, scales, zeros


def linear_plan(M: int, K: int, N: int, group: int = 128, plan=None) -> dict:
    p = _plan(plan) or Plan()
    _check(library().awq_linear_plan(M, K, N, group, ctypes.byref(p)))
    return {"path": p.path, "split_k": p.split_k, "waves": p.waves, "tpw": p.tpw, "x_stage": p.x_stage, "tile": p.tile}


def linear_workspace_bytes(M: int, K: int, N: int, group: int = 128, plan=None) -> int:
    out = ctypes.c_size_t(0)
    p = _plan(plan)
    _check(library().awq_linear_workspace_bytes_ex(M, K, N, group, ctypes.byref(p) if p else None,
                                                   ctypes.byref(out)))
    return int(out.value)


class Workspace:
    """A device buffer reused across calls on one stream (fp32 partial sums of
    split-K prefill plans; the library writes every byte it reads)."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        torch = _torch()
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def linear(x, qweight, scales, zeros, N: int, group: int = 128, out=None, workspace=None, plan=None):
    """y[M, N] fp16 = x[M, K] fp16 . W, W from (qweight, scales, zeros)."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    _need(qweight, torch.int32, "qweight")
    _need(scales, torch.float16, "scales", 2)
    _need(zeros, torch.int32, "zeros", 2)
    M, K = x.shape
    if scales.shape != (K // group, N) or zeros.shape != (K // group, N // 8):
        raise ValueError("scales must be [K/G, N] and zeros [K/G, N/8]")
    if qweight.numel() < qweight_words(K, N):
        raise ValueError("qweight is smaller than the device layout needs")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out", 2)
    p = _plan(plan)
    nbytes = linear_workspace_bytes(M, K, N, group, p)
    ws_ptr, ws_len = None, 0
    if nbytes:
        if workspace is None:
            workspace = Workspace(x.device)
        buf = workspace.get(nbytes) if isinstance(workspace, Workspace) else workspace
        ws_ptr, ws_len = buf.data_ptr(), buf.numel() * buf.element_size()
    lib = library()
    st = _stream(x.device)
    if p is None:
        status = lib.awq_linear(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), M, K, N,
                                group, out.data_ptr(), ws_ptr, ws_len, st)
    else:
        status = lib.awq_linear_ex(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), M, K, N,
                                   group, out.data_ptr(), ws_ptr, ws_len, ctypes.byref(p), st)
    _check(status)
    return out


def linear_noalloc(x, qweight, scales, zeros, N: int, group: int = 128, out=None, plan=None):
    """awq_linear without a workspace: split-K partials go to the library's
    own 64 MiB device array (nothing is allocated by the library; ``out`` may
    be passed in so that this call allocates nothing either)."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    _need(qweight, torch.int32, "qweight")
    _need(scales, torch.float16, "scales", 2)
    _need(zeros, torch.int32, "zeros", 2)
    M, K = x.shape
    if scales.shape != (K // group, N) or zeros.shape != (K // group, N // 8):
        raise ValueError("scales must be [K/G, N] and zeros [K/G, N/8]")
    if qweight.numel() < qweight_words(K, N):
        raise ValueError("qweight is smaller than the device layout needs")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out", 2)
    p = _plan(plan)
    _check(library().awq_linear_noalloc(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), M, K,
                                        N, group, out.data_ptr(), ctypes.byref(p) if p else None, _stream(x.device)))
    return out


def linear_silu_mul_plan(M: int, K: int, N: int, group: int = 128, plan=None) -> dict:
    p = _plan(plan) or Plan()
    _check(library().awq_linear_silu_mul_plan(M, K, N, group, ctypes.byref(p)))
    return {"path": p.path, "split_k": p.split_k, "waves": p.waves, "tpw": p.tpw, "x_stage": p.x_stage,
            "tile": p.tile}


def linear_silu_mul_workspace_bytes(M: int, K: int, N: int, group: int = 128, plan=None) -> int:
    out = ctypes.c_size_t()
    p = _plan(plan)
    _check(library().awq_linear_silu_mul_workspace_bytes(M, K, N, group, ctypes.byref(p) if p else None,
                                                         ctypes.byref(out)))
    return int(out.value)


def linear_silu_mul(x, qweight, scales, zeros, N: int, group: int = 128, out=None, workspace=None, plan=None):
    """y[M, N/2] fp16 = silu(g) * u with [g | u] = x . W (W's first N/2
    columns are the gate projection, the last N/2 the up projection)."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    _need(qweight, torch.int32, "qweight")
    _need(scales, torch.float16, "scales", 2)
    _need(zeros, torch.int32, "zeros", 2)
    M, K = x.shape
    if scales.shape != (K // group, N) or zeros.shape != (K // group, N // 8):
        raise ValueError("scales must be [K/G, N] and zeros [K/G, N/8]")
    if qweight.numel() < qweight_words(K, N):
        raise ValueError("qweight is smaller than the device layout needs")
    if out is None:
        out = torch.empty((M, N // 2), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out", 2)
    p = _plan(plan)
    nbytes = linear_silu_mul_workspace_bytes(M, K, N, group, p)
    ws_ptr, ws_len = None, 0
    if nbytes:
        if workspace is None:
            workspace = Workspace(x.device)
        buf = workspace.get(nbytes) if isinstance(workspace, Workspace) else workspace
        ws_ptr, ws_len = buf.data_ptr(), buf.numel() * buf.element_size()
    _check(library().awq_linear_silu_mul_ex(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                            M, K, N, group, out.data_ptr(), ws_ptr, ws_len,
                                            ctypes.byref(p) if p else None, _stream(x.device), None, None))
    return out


def quantize_act_fp8(x):
    """Per-token FP8 (E4M3) quantisation of fp16 x [M, K] (K % 128 == 0):
    returns (codes uint8 [M, K] in the kernel's layout -- within each
    128-column block, 8-column chunk 4j + h stored at position 4h + j -- and
    scales float32 [M])."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    M, K = x.shape
    x8 = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    sx = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(library().awq_quantize_act_fp8(x.data_ptr(), M, K, x8.data_ptr(), sx.data_ptr(), _stream(x.device)))
    return x8, sx


def linear_w4a8_plan(M: int, K: int, N: int, group: int = 128, plan=None) -> dict:
    p = _plan(plan) or Plan()
    _check(library().awq_linear_w4a8_plan(M, K, N, group, ctypes.byref(p)))
    return {"path": p.path, "split_k": p.split_k, "tile": p.tile}


def linear_w4a8_workspace_bytes(M: int, K: int, N: int, group: int = 128, plan=None) -> int:
    out = ctypes.c_size_t()
    p = _plan(plan)
    _check(library().awq_linear_w4a8_workspace_bytes(M, K, N, group, ctypes.byref(p) if p else None,
                                                     ctypes.byref(out)))
    return int(out.value)


def linear_w4a8(x, qweight, scales, zeros, N: int, group: int = 128, out=None, workspace=None, plan=None):
    """W4A8-FP8 layer: y[M, N] fp16 from fp16 x (quantised per token to FP8
    inside the call) and the layer's int4 weights; group a multiple of 128."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    _need(qweight, torch.int32, "qweight")
    _need(scales, torch.float16, "scales", 2)
    _need(zeros, torch.int32, "zeros", 2)
    M, K = x.shape
    if scales.shape != (K // group, N) or zeros.shape != (K // group, N // 8):
        raise ValueError("scales must be [K/G, N] and zeros [K/G, N/8]")
    if qweight.numel() < qweight_words(K, N):
        raise ValueError("qweight is smaller than the device layout needs")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out", 2)
    p = _plan(plan)
    nbytes = linear_w4a8_workspace_bytes(M, K, N, group, p)
    ws_ptr, ws_len = None, 0
    if nbytes:
        if workspace is None:
            workspace = Workspace(x.device)
        buf = workspace.get(nbytes) if isinstance(workspace, Workspace) else workspace
        ws_ptr, ws_len = buf.data_ptr(), buf.numel() * buf.element_size()
    _check(library().awq_linear_w4a8_ex(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), M, K,
                                        N, group, out.data_ptr(), ws_ptr, ws_len, ctypes.byref(p) if p else None,
                                        _stream(x.device), None, None))
    return out


def attention_desc(B: int, q_heads: int, kv_heads: int, head_dim: int, capacity: int, max_cached: int,
                   qkv_stride: int = 0, rope: str = "half", theta: float = 10000.0, scale: float = 0.0,
                   steps: int = 0) -> AttnDesc:
    """Descriptor of a fused decode-step attention call (see ``attention``)."""
    if rope not in ROPE_STYLES:
        raise ValueError(f"rope must be one of {sorted(ROPE_STYLES)}")
    d = AttnDesc()
    d.batch, d.q_heads, d.kv_heads, d.head_dim = B, q_heads, kv_heads, head_dim
    d.capacity, d.max_cached = capacity, max_cached
    d.qkv_stride = qkv_stride or (q_heads + 2 * kv_heads) * head_dim
    d.rope_style, d.steps = ROPE_STYLES[rope], steps
    d.rope_theta, d.softmax_scale = theta, scale
    return d


def attention_workspace_bytes(desc: AttnDesc) -> int:
    out = ctypes.c_size_t()
    _check(library().awq_attention_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return int(out.value)


def attention_plan(desc: AttnDesc) -> dict:
    c, s = ctypes.c_int32(), ctypes.c_int32()
    _check(library().awq_attention_plan(ctypes.byref(desc), ctypes.byref(c), ctypes.byref(s)))
    return {"workgroups_per_unit": int(c.value), "steps": int(s.value)}


class AttentionWorkspace:
    """Zero-filled device buffer for ``attention`` calls on one stream. The
    kernel returns its counters to zero, so the buffer is filled once, when it
    is allocated or grown."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def kv_cache(B: int, kv_heads: int, capacity: int, head_dim: int, device=None):
    """Zero-filled key cache [B, Hkv, capacity, D] and value cache
    [B, Hkv, capacity/32, D, 32] (tiles of 32 positions, d-major inside a
    tile), fp16, in the layouts ``attention`` reads."""
    torch = _torch()
    if capacity % 32:
        raise ValueError("capacity must be a multiple of 32")
    k = torch.zeros((B, kv_heads, capacity, head_dim), dtype=torch.float16, device=device)
    v = torch.zeros((B, kv_heads, capacity // 32, head_dim, 32), dtype=torch.float16, device=device)
    return k, v


def attention(qkv, k_cache, v_cache, lengths, q_heads: int, kv_heads: int, max_cached=None, rope: str = "half",
              theta: float = 10000.0, scale: float = 0.0, out=None, workspace=None, steps: int = 0, events=None):
    """One generation step of attention with the rotary embedding fused in.

    qkv [B, >= (Hq + 2 Hkv) D] fp16 (rows [q heads | k heads | v heads]),
    k_cache [B, Hkv, S, D] and v_cache [B, Hkv, S/32, D, 32] fp16 (see
    ``kv_cache``; updated in place:
    slot lengths[b] receives the new rotated key and the value), lengths [B]
    int32 on the device (tokens already cached). Returns out [B, Hq * D] fp16.
    ``max_cached`` bounds lengths on the host (default S - 1)."""
    torch = _torch()
    _need(k_cache, torch.float16, "k_cache", 4)
    _need(v_cache, torch.float16, "v_cache", 5)
    _need(lengths, torch.int32, "lengths", 1)
    if not isinstance(qkv, torch.Tensor) or qkv.dtype != torch.float16 or not qkv.is_cuda or qkv.dim() != 2:
        raise TypeError("qkv must be a 2-D fp16 GPU tensor")
    if qkv.stride(1) != 1:
        raise ValueError("qkv rows must be contiguous")
    B, Hkv, S, D = k_cache.shape
    if Hkv != kv_heads or S % 32 or v_cache.shape != (B, Hkv, S // 32, D, 32):
        raise ValueError("k_cache must be [B, Hkv, S, D] and v_cache [B, Hkv, S/32, D, 32]")
    if qkv.shape[0] != B or lengths.shape[0] != B or qkv.shape[1] < (q_heads + 2 * kv_heads) * D:
        raise ValueError("qkv must be [B, >= (Hq + 2 Hkv) D] and lengths [B]")
    desc = attention_desc(B, q_heads, kv_heads, D, S, S - 1 if max_cached is None else int(max_cached),
                          qkv.stride(0) if B > 1 else qkv.shape[1] + (-qkv.shape[1]) % 8, rope, theta, scale,
                          steps)
    if out is None:
        out = torch.empty((B, q_heads * D), dtype=torch.float16, device=qkv.device)
    else:
        _need(out, torch.float16, "out", 2)
        if out.shape != (B, q_heads * D):
            raise ValueError("out must be [B, Hq * D]")
    nbytes = attention_workspace_bytes(desc)
    if workspace is None:
        workspace = AttentionWorkspace(qkv.device)
    buf = workspace.get(nbytes) if isinstance(workspace, AttentionWorkspace) else workspace
    lib = library()
    args = (ctypes.byref(desc), qkv.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lengths.data_ptr(),
            out.data_ptr(), buf.data_ptr(), buf.numel() * buf.element_size(), _stream(qkv.device))
    if events is None:
        _check(lib.awq_attention_decode(*args))
    else:
        _check(lib.awq_attention_decode_timed(*args, events[0], events[1]))
    return out


__all__ = ["quantize_act_fp8", "linear_w4a8", "linear_w4a8_plan", "linear_w4a8_workspace_bytes", "attention", "attention_desc", "attention_plan", "attention_workspace_bytes", "kv_cache",
           "AttentionWorkspace", "library", "pack", "unpack", "pack_zeros", "dequant", "quantize", "linear", "linear_silu_mul",
           "linear_silu_mul_plan", "linear_silu_mul_workspace_bytes", "linear_plan", "linear_noalloc",
           "linear_workspace_bytes", "qweight_words", "Plan", "Workspace", "AWQError", "AWQLibraryMissing",
           "abi_version"]
