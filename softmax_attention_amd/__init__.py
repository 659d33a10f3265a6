"""Python binding of libhla (hybrid linear-softmax attention on gfx950).

A thin ctypes layer over the C ABI in include/hla.h, with the same names:
``hla_linear_fwd``, ``hla_softmax_anchor_fwd``, ``hla_hybrid_stack_fwd``,
``hla_linear_workspace_bytes``, ``hla_status_str``, ``hla_abi_version``,
``hla_linear_write_gated_fwd`` and ``hla_attnres_route_fwd``. It only
marshals arguments: torch tensors become device pointers and the current torch
stream becomes the HIP stream; every step of the computation runs in the HIP
kernels. The shared library must have been built (``python
softmax_attention_amd/build.py``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhla.so")

HLA_F32 = 0
HLA_BF16 = 1
HLA_FP8_E4M3 = 2
HLA_LAYER_LINEAR = 0
HLA_LAYER_SOFTMAX = 1
STATUS = {
    0: "HLA_OK", 1: "HLA_ERR_NULL_PTR", 2: "HLA_ERR_BAD_SHAPE", 3: "HLA_ERR_UNSUPPORTED",
    4: "HLA_ERR_BAD_ARG", 5: "HLA_ERR_ALIGN", 6: "HLA_ERR_WORKSPACE", 7: "HLA_ERR_HIP",
}
EXPORTS = ("hla_abi_version", "hla_status_str", "hla_linear_workspace_bytes", "hla_linear_fwd",
           "hla_linear_fwd_noalloc", "hla_linear_write_gated_fwd", "hla_softmax_anchor_workspace_bytes",
           "hla_softmax_anchor_fwd", "hla_softmax_anchor_fp8p_fwd", "hla_hybrid_stack_fwd",
           "hla_attnres_route_fwd")


class hla_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("D", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class HLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


def hip_runtimes_loaded() -> list:
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            maps = f.read()
    except OSError:
        return []
    return sorted({line.split()[-1] for line in maps.splitlines()
                   if "libamdhip64" in line and "/" in line})


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python softmax_attention_amd/build.py`")
    # torch ships its own HIP runtime. Load it first so that libhla binds to that
    # same runtime (same soname) instead of pulling in a second copy from
    # /opt/rocm: device memory and streams come from torch, and two runtimes in
    # one process cannot share them.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = hip_runtimes_loaded()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime is loaded: {runtimes}")
    P = ctypes.c_void_p
    pd = ctypes.POINTER(hla_dims)
    lib.hla_abi_version.restype = ctypes.c_int
    lib.hla_abi_version.argtypes = []
    lib.hla_status_str.restype = ctypes.c_char_p
    lib.hla_status_str.argtypes = [ctypes.c_int]
    lib.hla_linear_workspace_bytes.restype = ctypes.c_size_t
    lib.hla_linear_workspace_bytes.argtypes = [pd]
    lib.hla_linear_fwd.restype = ctypes.c_int
    lib.hla_linear_fwd.argtypes = [pd, P, P, P, P, P, ctypes.c_int, ctypes.c_float, P,
                                   ctypes.c_size_t, P]
    lib.hla_linear_fwd_noalloc.restype = ctypes.c_int
    lib.hla_linear_fwd_noalloc.argtypes = [pd, P, P, P, P, P, ctypes.c_int, ctypes.c_float, P]
    lib.hla_linear_write_gated_fwd.restype = ctypes.c_int
    lib.hla_linear_write_gated_fwd.argtypes = [pd, P, P, P, P, P, P, ctypes.c_int, ctypes.c_float,
                                               P, ctypes.c_size_t, P]
    lib.hla_softmax_anchor_workspace_bytes.restype = ctypes.c_size_t
    lib.hla_softmax_anchor_workspace_bytes.argtypes = [pd]
    lib.hla_softmax_anchor_fwd.restype = ctypes.c_int
    lib.hla_softmax_anchor_fwd.argtypes = [pd, P, P, P, P, P, ctypes.c_int, ctypes.c_float, P,
                                           ctypes.c_size_t, P]
    lib.hla_softmax_anchor_fp8p_fwd.restype = ctypes.c_int
    lib.hla_softmax_anchor_fp8p_fwd.argtypes = [pd, P, P, P, P, P, ctypes.c_int, ctypes.c_float, P,
                                                ctypes.c_size_t, P]
    lib.hla_hybrid_stack_fwd.restype = ctypes.c_int
    lib.hla_hybrid_stack_fwd.argtypes = [pd, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                         ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                                         ctypes.POINTER(P), P, ctypes.c_float, ctypes.c_float, P,
                                         ctypes.c_size_t, P]
    lib.hla_attnres_route_fwd.restype = ctypes.c_int
    lib.hla_attnres_route_fwd.argtypes = [pd, ctypes.c_int, ctypes.POINTER(P), P, P, P, P]
    return lib


lib = _load()


def hla_abi_version() -> int:
    return lib.hla_abi_version()


def hla_status_str(status: int) -> str:
    return lib.hla_status_str(status).decode()


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    """hla_dtype of a torch dtype (or of a tensor's dtype)."""
    torch = _torch()
    dt = getattr(dt, "dtype", dt)
    if dt == torch.float32:
        return HLA_F32
    if dt == torch.bfloat16:
        return HLA_BF16
    if dt == torch.float8_e4m3fn:
        return HLA_FP8_E4M3
    raise TypeError(f"unsupported dtype {dt}")


def dims_of(q, out_dtype=None) -> hla_dims:
    """hla_dims of a [B, H, N, D] tensor.

    out_dtype defaults to the output dtype a call makes when given no output:
    q's dtype, except bf16 for fp8 inputs (fp8 outputs are not built)."""
    if q.dim() != 4:
        raise ValueError(f"expected [B, H, N, D], got shape {tuple(q.shape)}")
    B, H, N, D = (int(x) for x in q.shape)
    ind = _dtype_code(q)
    if out_dtype is None:
        outd = HLA_BF16 if ind == HLA_FP8_E4M3 else ind
    else:
        outd = _dtype_code(out_dtype)
    return hla_dims(B, H, N, D, ind, outd)


def _new_out(q):
    """Default output: q's dtype, except bf16 for fp8 inputs (fp8 outputs are not built)."""
    torch = _torch()
    return torch.empty_like(q, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn else None)


def _check(*ts):
    """Inputs of one call: on the GPU, on one device, contiguous, one shape, one dtype.

    The C ABI takes a single in_dtype (from q) for q, k, v and g; a tensor of another
    dtype would be read with the wrong element size, so the mismatch is refused here,
    before any launch."""
    ref = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t.device != ref.device:
            raise ValueError(f"tensors on different devices: {t.device} vs {ref.device}")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, D]")
        if t.shape != ref.shape:
            raise ValueError(f"shape mismatch {tuple(t.shape)} vs {tuple(ref.shape)}")
        if t.dtype != ref.dtype:
            raise ValueError(f"dtype mismatch {t.dtype} vs {ref.dtype}: q, k, v and g share one dtype")


def _check_out(q, out):
    """The output (or residual stream) of a call: q's shape and device, contiguous."""
    if not out.is_cuda or out.device != q.device:
        raise ValueError(f"out must live on q's device {q.device}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous [B, H, N, D]")
    if out.shape != q.shape:
        raise ValueError(f"shape mismatch {tuple(out.shape)} vs {tuple(q.shape)}")


def _stream(stream, device) -> int:
    """HIP stream handle of the call: ``stream``, or torch's current stream on ``device``."""
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return int(s.cuda_stream)


def _on(stream, device):
    """Context for a call's allocations and launch: the tensors' device, and the call's
    stream as torch's current stream, so that a workspace or output allocated here
    belongs to the stream that uses it (the caching allocator hands a freed block only
    to later work on the same stream)."""
    import contextlib
    torch = _torch()
    ctx = contextlib.ExitStack()
    ctx.enter_context(torch.cuda.device(device))
    if stream is not None:
        ctx.enter_context(torch.cuda.stream(stream))
    return ctx


def _raise(fn: str, st: int):
    if st != 0:
        if st == 7:
            # some launches may already be queued: let them finish before the
            # caller's tensors can be freed
            _torch().cuda.synchronize()
        raise HLAError(fn, st)


def hla_linear_workspace_bytes(dims: hla_dims) -> int:
    return int(lib.hla_linear_workspace_bytes(ctypes.byref(dims)))


def hla_softmax_anchor_workspace_bytes(dims: hla_dims) -> int:
    return int(lib.hla_softmax_anchor_workspace_bytes(ctypes.byref(dims)))


def _workspace(nbytes: int, device):
    return _torch().empty(max(int(nbytes), 256), dtype=_torch().uint8, device=device)


def linear_workspace(q, out_dtype=None):
    """A device workspace tensor sized for hla_linear_fwd on q's shape."""
    return _workspace(hla_linear_workspace_bytes(dims_of(q, out_dtype)), q.device)


def anchor_workspace(q, out_dtype=None):
    """A device workspace tensor sized for hla_softmax_anchor_fwd on q's shape."""
    return _workspace(hla_softmax_anchor_workspace_bytes(dims_of(q, out_dtype)), q.device)


def stack_workspace(q, kinds, out_dtype=None):
    """A device workspace tensor sized for hla_hybrid_stack_fwd with these layer kinds."""
    d = dims_of(q, out_dtype)
    n = 0
    if any(k == HLA_LAYER_LINEAR for k in kinds):
        n = max(n, hla_linear_workspace_bytes(d))
    if any(k == HLA_LAYER_SOFTMAX for k in kinds):
        n = max(n, hla_softmax_anchor_workspace_bytes(d))
    return _workspace(n, q.device)


def _workspace_check(workspace, q):
    if not workspace.is_cuda or workspace.device != q.device:
        raise ValueError(f"workspace must live on q's device {q.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def hla_linear_fwd(q, k, v, g, out=None, accumulate: bool = False, eps: float = 1e-6,
                   workspace=None, stream=None):
    """Gated linear attention O = sigma(G) * (phi(Q) S) / (phi(Q) z + eps); returns out."""
    _check(q, k, v, g)
    if out is not None:
        _check_out(q, out)
    with _on(stream, q.device):
        if out is None:
            out = _new_out(q)
        d = dims_of(q, out.dtype)
        if workspace is None:
            workspace = linear_workspace(q, out.dtype)
        _workspace_check(workspace, q)
        st = lib.hla_linear_fwd(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                g.data_ptr(), out.data_ptr(), int(bool(accumulate)), float(eps),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream(stream, q.device))
    _raise("hla_linear_fwd", st)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # HLA_NOALLOC_SCRATCH_BYTES of include/hla.h


def hla_linear_fwd_noalloc(q, k, v, g, out, accumulate: bool = False, eps: float = 1e-6,
                           stream=None):
    """hla_linear_fwd without a workspace: the library's per-GPU scratch array holds
    the partial states. The caller passes the output; nothing is allocated."""
    _check(q, k, v, g)
    _check_out(q, out)
    with _on(stream, q.device):
        d = dims_of(q, out.dtype)
        st = lib.hla_linear_fwd_noalloc(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        g.data_ptr(), out.data_ptr(), int(bool(accumulate)),
                                        float(eps), _stream(stream, q.device))
    _raise("hla_linear_fwd_noalloc", st)
    return out


def hla_linear_write_gated_fwd(q, k, v, g, w, out=None, accumulate: bool = False,
                               eps: float = 1e-6, workspace=None, stream=None):
    """Write-gated linear attention: token n enters the state with sigma(w_n); returns out.

    w has shape [B, H, N] and the dtype of q."""
    _check(q, k, v, g)
    if tuple(w.shape) != tuple(q.shape[:-1]) or w.dtype != q.dtype or not w.is_contiguous():
        raise ValueError("w must be a contiguous [B, H, N] tensor of q's dtype")
    if not w.is_cuda or w.device != q.device:
        raise ValueError(f"w must live on q's device {q.device}")
    if out is not None:
        _check_out(q, out)
    with _on(stream, q.device):
        if out is None:
            out = _new_out(q)
        d = dims_of(q, out.dtype)
        if workspace is None:
            workspace = linear_workspace(q, out.dtype)
        _workspace_check(workspace, q)
        st = lib.hla_linear_write_gated_fwd(ctypes.byref(d), q.data_ptr(), k.data_ptr(),
                                            v.data_ptr(), g.data_ptr(), w.data_ptr(),
                                            out.data_ptr(), int(bool(accumulate)), float(eps),
                                            workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(stream, q.device))
    _raise("hla_linear_write_gated_fwd", st)
    return out


def hla_softmax_anchor_fwd(q, k, v, g, out=None, accumulate: bool = False,
                           scale: Optional[float] = None, workspace=None, stream=None):
    """Gated softmax anchor O = sigma(G) * softmax(scale Q K^T) V; returns out."""
    return _anchor("hla_softmax_anchor_fwd", q, k, v, g, out, accumulate, scale, workspace, stream)


def hla_softmax_anchor_fp8p_fwd(q, k, v, g, out=None, accumulate: bool = False,
                                scale: Optional[float] = None, workspace=None, stream=None):
    """The gated softmax anchor on fp8 (e4m3) inputs with probabilities rounded to
    e4m3 and P V on the fp8 matrix cores; returns out."""
    if _dtype_code(q) != HLA_FP8_E4M3:
        raise TypeError("hla_softmax_anchor_fp8p_fwd takes float8_e4m3fn inputs")
    return _anchor("hla_softmax_anchor_fp8p_fwd", q, k, v, g, out, accumulate, scale, workspace,
                   stream)


def _anchor(name, q, k, v, g, out, accumulate, scale, workspace, stream):
    _check(q, k, v, g)
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    if out is not None:
        _check_out(q, out)
    with _on(stream, q.device):
        if out is None:
            out = _new_out(q)
        d = dims_of(q, out.dtype)
        if workspace is None:
            workspace = anchor_workspace(q, out.dtype)
        _workspace_check(workspace, q)
        st = getattr(lib, name)(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                g.data_ptr(), out.data_ptr(), int(bool(accumulate)), scale,
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream(stream, q.device))
    _raise(name, st)
    return out


def hla_hybrid_stack_fwd(x, layers: Sequence, kinds: Sequence[int], eps: float = 1e-6,
                         scale: Optional[float] = None, workspace=None, stream=None):
    """x += layer_l(q_l, k_l, v_l, g_l) for each layer in order (in place); returns x.

    Every layer's q, k, v, g share the shape, dtype and device of layer 0's q."""
    n = len(layers)
    if n != len(kinds):
        raise ValueError("layers and kinds differ in length")
    if n == 0:
        raise ValueError("the stack needs at least one layer")
    q0 = layers[0][0]
    for (q, k, v, g) in layers:
        _check(q0, q, k, v, g)
    _check_out(q0, x)
    scale = 1.0 / math.sqrt(q0.shape[-1]) if scale is None else float(scale)
    with _on(stream, q0.device):
        d = dims_of(q0, x.dtype)
        if workspace is None:
            workspace = stack_workspace(q0, kinds, x.dtype)
        _workspace_check(workspace, q0)
        arr = ctypes.c_void_p * n
        qs = arr(*[l[0].data_ptr() for l in layers])
        ks = arr(*[l[1].data_ptr() for l in layers])
        vs = arr(*[l[2].data_ptr() for l in layers])
        gs = arr(*[l[3].data_ptr() for l in layers])
        kd = (ctypes.c_int32 * n)(*[int(x_) for x_ in kinds])
        st = lib.hla_hybrid_stack_fwd(ctypes.byref(d), n, kd, qs, ks, vs, gs, x.data_ptr(),
                                      float(eps), scale, workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream, q0.device))
    _raise("hla_hybrid_stack_fwd", st)
    return x


def hla_attnres_route_fwd(x, summaries: Sequence, w, out=None, stream=None):
    """Routed residual stream x + sum_i softmax_i((x W) . s_i / sqrt(D)) s_i; returns out.

    x and every summary: fp32 [B, H, N, D] on the GPU; w: bf16 [D, D] router
    projection shared across depth; out defaults to a new tensor (pass x to route
    in place)."""
    torch = _torch()
    _check(x, *summaries)
    if x.dtype != torch.float32:
        raise ValueError("x and the summaries must be fp32")
    D = int(x.shape[-1])
    if (tuple(w.shape) != (D, D) or w.dtype != torch.bfloat16 or not w.is_contiguous()
            or not w.is_cuda or w.device != x.device):
        raise ValueError("w must be a contiguous bf16 [D, D] tensor on x's device")
    if out is not None:
        _check_out(x, out)
        if out.dtype != torch.float32:
            raise ValueError("out must be fp32")
    with _on(stream, x.device):
        if out is None:
            out = torch.empty_like(x)
        d = dims_of(x, out.dtype)
        n = len(summaries)
        arr = (ctypes.c_void_p * max(n, 1))(*[s_.data_ptr() for s_ in summaries])
        st = lib.hla_attnres_route_fwd(ctypes.byref(d), n, arr, x.data_ptr(), w.data_ptr(),
                                       out.data_ptr(), _stream(stream, x.device))
    _raise("hla_attnres_route_fwd", st)
    return out
