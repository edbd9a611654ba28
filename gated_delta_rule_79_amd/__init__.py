"""Kimi Delta Attention on MI355X (gfx950): Python binding of libkda.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so (see include/kda.h for the C ABI).  PyTorch supplies
device memory and the current stream.  If the library is not built this
module raises on use; there is no fallback implementation.

    o, S_T = fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None)
    dq, dk, dv, dlog_alpha, dbeta, d_init = bwd(q, k, v, log_alpha, beta, d_out, ...)
    out = decode(q, k, v, log_alpha, beta, state_pool, state_indices, num_commit)
    y, conv_state = conv_fwd(x, weight, bias, init_state, cu_seqlens, silu=True)   # short convolution

Shapes: q, k, log_alpha [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H]; all of
one dtype (torch.float32 or torch.bfloat16), contiguous, on the GPU.  States
are float32 [N, H, dk, dv] with N = B, or N = len(cu_seqlens) - 1 for a packed
varlen batch (then B must be 1 and cu_seqlens is int32 on the GPU).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "bwd", "decode", "workspace_bytes", "conv_fwd", "conv_bwd", "conv_decode", "conv_workspace_bytes",
           "KdaError", "lib_path", "load_library", "status_string", "timing_enable", "timing_read"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None

KDA_F32, KDA_BF16 = 0, 1
KDA_ERROR_LAUNCH = 5   # kda_status value of a failed kernel launch (include/kda.h)
KDA_FLAG_SAVE_FOR_BACKWARD, KDA_FLAG_USE_SAVED = 1, 2   # kda_desc.flags bits (include/kda.h)
KDA_FLAG_QK_L2NORM, KDA_FLAG_GATE_LOGSIGMOID = 4, 8     # fused input preparation


def _prep_flags(qk_l2norm, gate_logsigmoid):
    return (KDA_FLAG_QK_L2NORM if qk_l2norm else 0) | (KDA_FLAG_GATE_LOGSIGMOID if gate_logsigmoid else 0)


class kda_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("flags", ctypes.c_int32)]


class kda_conv_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("W", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("activation", ctypes.c_int32)]


KDA_CONV_IDENTITY, KDA_CONV_SILU = 0, 1


class KdaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        detail = last_error() if status == KDA_ERROR_LAUNCH or fn == "kda_fwd_noalloc" else ""
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})" + (f": {detail}" if detail else ""))


def lib_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libkda.so not found at {p}; build it with gated_delta_rule_79_amd.build.build()")
    # torch ships its own HIP runtime; loading torch first makes libkda.so bind to
    # that same runtime (a second runtime in the process cannot see the device
    # memory and streams torch hands over).
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    D = ctypes.POINTER(kda_desc)
    lib.kda_workspace_bytes.argtypes = [D, ctypes.c_int]
    lib.kda_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_decode.argtypes = [D, P, P, P, P, P, P, ctypes.c_int32, P, P, P, P]
    lib.kda_decode.restype = ctypes.c_int
    CD = ctypes.POINTER(kda_conv_desc)
    lib.kda_conv_workspace_bytes.argtypes = [CD]
    lib.kda_conv_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_conv_fwd.argtypes = [CD, P, P, P, P, P, P, P, P]
    lib.kda_conv_fwd.restype = ctypes.c_int
    lib.kda_conv_bwd.argtypes = [CD, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_conv_bwd.restype = ctypes.c_int
    lib.kda_conv_decode.argtypes = [CD, P, P, P, P, ctypes.c_int32, P, P, P, P]
    lib.kda_conv_decode.restype = ctypes.c_int
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_timing_enable.argtypes = [ctypes.c_int]
    lib.kda_timing_enable.restype = None
    lib.kda_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int)]
    lib.kda_timing_read.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def timing_enable(on: bool = True) -> None:
    """Record a HIP event pair around every later kernel launch (clears totals when enabling)."""
    load_library().kda_timing_enable(1 if on else 0)


def timing_read() -> dict:
    """{kernel name: (total milliseconds, launches)} of the launches recorded so far (waits for them)."""
    lib = load_library()
    n = 64
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    k = lib.kda_timing_read(n, names, ms, cnt)
    if k < 0:
        raise RuntimeError("kda_timing_read: a HIP event call failed")
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(k)}


def status_string(status: int) -> str:
    try:
        return load_library().kda_status_string(int(status)).decode()
    except Exception:  # library missing: still give a readable message
        return f"status {status}"


def last_error() -> str:
    """The failing kernel launch and HIP error of this thread's last kda_fwd/kda_bwd call ("" if none)."""
    try:
        return load_library().kda_last_error().decode()
    except Exception:  # library missing
        return ""


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def make_desc(B, T, H, dk, dv, dtype_code, num_seqs=0, scale=None, out_code=KDA_F32, flags=0) -> kda_desc:
    return kda_desc(int(B), int(T), int(H), int(dk), int(dv), int(num_seqs), int(dtype_code), int(out_code),
                    float(scale) if scale else 0.0, int(flags))


def workspace_bytes(B, T, H, dk, dv, dtype, num_seqs=0, backward=False, qk_l2norm=False,
                    gate_logsigmoid=False) -> int:
    import torch
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    d = make_desc(B, T, H, dk, dv, code, num_seqs, flags=_prep_flags(qk_l2norm, gate_logsigmoid))
    return int(load_library().kda_workspace_bytes(ctypes.byref(d), 1 if backward else 0))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _prepare(q, k, v, log_alpha, beta, init_state, cu_seqlens, scale, out_dtype=None):
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    dt = q.dtype
    _check("k", k, dt, (B, T, H, dk), dev)
    _check("log_alpha", log_alpha, dt, (B, T, H, dk), dev)
    _check("v", v, dt, (B, T, H, dv), dev)
    _check("beta", beta, dt, (B, T, H), dev)
    _check("q", q, dt, (B, T, H, dk), dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
            raise ValueError("cu_seqlens must be int32 [N+1] on the GPU")
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    if init_state is not None:
        _check("init_state", init_state, torch.float32, (N, H, dk, dv), dev)
    odt = torch.float32 if out_dtype is None else out_dtype
    desc = make_desc(B, T, H, dk, dv, _dtype_code(dt), N if cu_seqlens is not None else 0, scale, _dtype_code(odt))
    return desc, (B, T, H, dk, dv, N), dev, odt


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def fwd(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, scale=None, output_final_state=True,
        out=None, final_state=None, workspace=None, out_dtype=None, save_for_backward=False, qk_l2norm=False,
        gate_logsigmoid=False):
    """Forward pass; returns (o [B,T,H,dv] in out_dtype (default float32), final_state float32
    [N,H,dk,dv] or None).  out_dtype=torch.bfloat16 is allowed for bf16 inputs.
    save_for_backward=True leaves the backward's intermediates in `workspace` (which must then be
    given, sized by workspace_bytes(..., backward=True)) for a following bwd(..., use_saved=True).
    qk_l2norm / gate_logsigmoid: q, k arrive raw and are L2-normalised inside; log_alpha holds a raw
    gate x (log alpha = logsigmoid(x) inside)."""
    import torch
    lib = load_library()
    desc, (B, T, H, dk, dv, N), dev, dt = _prepare(q, k, v, log_alpha, beta, init_state, cu_seqlens, scale,
                                                   out_dtype)
    desc.flags = _prep_flags(qk_l2norm, gate_logsigmoid)
    if save_for_backward:
        if workspace is None:
            raise ValueError("save_for_backward needs the caller's workspace (it is reused by bwd)")
        desc.flags |= KDA_FLAG_SAVE_FOR_BACKWARD
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check("out", out, dt, (B, T, H, dv), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check("final_state", final_state, torch.float32, (N, H, dk, dv), dev)
    need = lib.kda_workspace_bytes(ctypes.byref(desc), 1 if save_for_backward else 0)
    if workspace is None or (not save_for_backward and workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state),
                     _ptr(out), _ptr(final_state), _ptr(cu_seqlens), _ptr(workspace),
                     workspace.numel() * workspace.element_size(), _stream(dev))
    if rc:
        raise KdaError("kda_fwd", rc)
    return out, final_state


NOALLOC_SCRATCH_BYTES = 128 << 20   # KDA_NOALLOC_SCRATCH_BYTES in kda.h


def fwd_noalloc(q, k, v, log_alpha, beta, out, final_state=None, init_state=None, cu_seqlens=None, scale=None,
                out_dtype=None, qk_l2norm=False, gate_logsigmoid=False):
    """kda_fwd_noalloc: the forward pass with the library's own device scratch as its
    workspace.  The caller passes out (and final_state, or None) already allocated;
    nothing is allocated here or in the library.  Returns (out, final_state)."""
    lib = load_library()
    desc, (B, T, H, dk, dv, N), dev, dt = _prepare(q, k, v, log_alpha, beta, init_state, cu_seqlens, scale,
                                                   out_dtype)
    desc.flags = _prep_flags(qk_l2norm, gate_logsigmoid)
    _check("out", out, dt, (B, T, H, dv), dev)
    if final_state is not None:
        import torch
        _check("final_state", final_state, torch.float32, (N, H, dk, dv), dev)
    rc = lib.kda_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                             _ptr(init_state), _ptr(out), _ptr(final_state), _ptr(cu_seqlens), _stream(dev))
    if rc:
        raise KdaError("kda_fwd_noalloc", rc)
    return out, final_state


def bwd(q, k, v, log_alpha, beta, d_out, init_state=None, d_final_state=None, cu_seqlens=None, scale=None,
        need_d_init=True, workspace=None, out_dtype=None, grads=None, d_init=None, use_saved=False,
        qk_l2norm=False, gate_logsigmoid=False):
    """Backward pass; returns (dq, dk, dv, dlog_alpha, dbeta in out_dtype (default float32),
    d_init_state float32 or None).  use_saved=True: `workspace` holds what fwd(...,
    save_for_backward=True) left there for the same inputs; the forward is not recomputed."""
    import torch
    lib = load_library()
    desc, (B, T, H, dk, dv, N), dev, odt = _prepare(q, k, v, log_alpha, beta, init_state, cu_seqlens, scale,
                                                    out_dtype)
    desc.flags = _prep_flags(qk_l2norm, gate_logsigmoid)
    if use_saved:
        if workspace is None:
            raise ValueError("use_saved needs the workspace the forward wrote")
        desc.flags |= KDA_FLAG_USE_SAVED
    _check("d_out", d_out, q.dtype, (B, T, H, dv), dev)
    if d_final_state is not None:
        _check("d_final_state", d_final_state, torch.float32, (N, H, dk, dv), dev)
    if grads is None:
        grads = tuple(torch.empty(x.shape, dtype=odt, device=dev) for x in (q, k, v, log_alpha, beta))
    for name, g, x in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta"), grads, (q, k, v, log_alpha, beta)):
        _check(name, g, odt, x.shape, dev)
    dq, dkk, dvv, dla, db = grads
    dinit = d_init
    if dinit is None and need_d_init:
        dinit = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif dinit is not None:
        _check("d_init", dinit, torch.float32, (N, H, dk, dv), dev)
    need = lib.kda_workspace_bytes(ctypes.byref(desc), 1)
    if workspace is None or (not use_saved and workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(init_state),
                     _ptr(cu_seqlens), _ptr(d_out), _ptr(d_final_state), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dla),
                     _ptr(db), _ptr(dinit), _ptr(workspace), workspace.numel() * workspace.element_size(),
                     _stream(dev))
    if rc:
        raise KdaError("kda_bwd", rc)
    return dq, dkk, dvv, dla, db, dinit


DECODE_MAX_TOKENS = 16   # KDA_DECODE_MAX_TOKENS (include/kda.h)


def decode(q, k, v, log_alpha, beta, state_pool, state_indices=None, num_commit=None, scale=None,
           out=None, out_dtype=None, qk_l2norm=False, gate_logsigmoid=False):
    """Decode / replay step: advance B sequences by T tokens each from states in `state_pool`.

    q, k, log_alpha [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H] (float32 or bfloat16);
    state_pool float32 [P,H,dk,dv], updated in place; state_indices int32 [B] (None: slot b;
    outside [0, P): padding); num_commit int32 [B] (None: T): the slot receives the state after
    that many tokens.  Returns out [B,T,H,dv] (every token's output, out_dtype default float32)."""
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    dt = q.dtype
    for name, t, shape in (("k", k, (B, T, H, dk)), ("log_alpha", log_alpha, (B, T, H, dk)),
                           ("v", v, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _check(name, t, dt, shape, dev)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [P, H, dk, dv]")
    _check("state_pool", state_pool, torch.float32, (state_pool.shape[0], H, dk, dv), dev)
    for name, t in (("state_indices", state_indices), ("num_commit", num_commit)):
        if t is not None:
            _check(name, t, torch.int32, (B,), dev)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=odt, device=dev)
    else:
        _check("out", out, odt, (B, T, H, dv), dev)
    desc = make_desc(B, T, H, dk, dv, _dtype_code(dt), 0, scale, _dtype_code(odt),
                     flags=_prep_flags(qk_l2norm, gate_logsigmoid))
    rc = lib.kda_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                        _ptr(state_pool), int(state_pool.shape[0]), _ptr(state_indices), _ptr(num_commit),
                        _ptr(out), _stream(dev))
    if rc:
        raise KdaError("kda_decode", rc)
    return out


# ---------------------------------------------------------------------------
# short causal convolution with a carried state (kda_conv_* in include/kda.h)
# ---------------------------------------------------------------------------
def _conv_desc(x, W, cu_seqlens, out_dtype, silu, decode=False):
    import torch
    if x.dim() != 3:
        raise ValueError("x must be [B, T, D]")
    B, T, D = x.shape
    if x.device.type != "cuda":
        raise ValueError("inputs must be on the GPU")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    N = B
    if cu_seqlens is not None:
        if decode or B != 1:
            raise ValueError("cu_seqlens requires B == 1 (and is not used by the decode step)")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != x.device:
            raise ValueError("cu_seqlens must be int32 [N+1] on the GPU")
        N = cu_seqlens.shape[0] - 1
    odt = torch.float32 if out_dtype is None else out_dtype
    d = kda_conv_desc(int(B), int(T), int(D), int(W), int(N) if cu_seqlens is not None else 0, _dtype_code(x.dtype),
                      _dtype_code(odt), KDA_CONV_SILU if silu else KDA_CONV_IDENTITY)
    return d, (B, T, D, N), odt


def _conv_params(weight, bias, D, dev):
    import torch
    if weight.dim() != 2 or weight.shape[0] != D:
        raise ValueError("weight must be float32 [D, W]")
    _check("weight", weight, torch.float32, (D, weight.shape[1]), dev)
    if bias is not None:
        _check("bias", bias, torch.float32, (D,), dev)
    return int(weight.shape[1])


def conv_workspace_bytes(B, T, D, W, dtype) -> int:
    """Workspace bytes of conv_bwd (partial sums of dweight and dbias)."""
    import torch
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    d = kda_conv_desc(int(B), int(T), int(D), int(W), 0, code, KDA_F32, 0)
    return int(load_library().kda_conv_workspace_bytes(ctypes.byref(d)))


def conv_fwd(x, weight, bias=None, init_state=None, cu_seqlens=None, silu=False, out=None, final_state=None,
             output_final_state=True, out_dtype=None):
    """Short causal convolution: x [B, T, D] (or packed [1, T, D] with cu_seqlens), weight float32 [D, W],
    bias float32 [D] or None, init_state float32 [N, W-1, D] or None.  Returns (y [B, T, D] in out_dtype
    (default float32), final_state float32 [N, W-1, D] or None)."""
    import torch
    lib = load_library()
    dev = x.device
    W = _conv_params(weight, bias, x.shape[-1], dev)
    desc, (B, T, D, N), odt = _conv_desc(x, W, cu_seqlens, out_dtype, silu)
    if init_state is not None:
        _check("init_state", init_state, torch.float32, (N, W - 1, D), dev)
    if out is None:
        out = torch.empty((B, T, D), dtype=odt, device=dev)
    else:
        _check("out", out, odt, (B, T, D), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, W - 1, D), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check("final_state", final_state, torch.float32, (N, W - 1, D), dev)
    rc = lib.kda_conv_fwd(ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(bias), _ptr(init_state), _ptr(out),
                          _ptr(final_state), _ptr(cu_seqlens), _stream(dev))
    if rc:
        raise KdaError("kda_conv_fwd", rc)
    return out, final_state


def conv_bwd(x, weight, dy, bias=None, init_state=None, d_final_state=None, cu_seqlens=None, silu=False,
             out_dtype=None, need_d_bias=True, need_d_init=True, workspace=None, dx=None, dweight=None,
             dbias=None, d_init=None):
    """Gradients of <dy, y> + <d_final_state, final_state>: returns (dx in out_dtype (default float32),
    dweight float32 [D, W], dbias float32 [D] or None, d_init_state float32 [N, W-1, D] or None)."""
    import torch
    lib = load_library()
    dev = x.device
    W = _conv_params(weight, bias, x.shape[-1], dev)
    desc, (B, T, D, N), odt = _conv_desc(x, W, cu_seqlens, out_dtype, silu)
    _check("dy", dy, x.dtype, (B, T, D), dev)
    for name, t in (("init_state", init_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check(name, t, torch.float32, (N, W - 1, D), dev)
    dx = torch.empty((B, T, D), dtype=odt, device=dev) if dx is None else dx
    _check("dx", dx, odt, (B, T, D), dev)
    dweight = torch.empty((D, W), dtype=torch.float32, device=dev) if dweight is None else dweight
    _check("dweight", dweight, torch.float32, (D, W), dev)
    if dbias is None and need_d_bias:
        dbias = torch.empty((D,), dtype=torch.float32, device=dev)
    if dbias is not None:
        _check("dbias", dbias, torch.float32, (D,), dev)
    if d_init is None and need_d_init:
        d_init = torch.empty((N, W - 1, D), dtype=torch.float32, device=dev)
    if d_init is not None:
        _check("d_init", d_init, torch.float32, (N, W - 1, D), dev)
    need = lib.kda_conv_workspace_bytes(ctypes.byref(desc))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_conv_bwd(ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(bias), _ptr(init_state),
                          _ptr(cu_seqlens), _ptr(dy), _ptr(d_final_state), _ptr(dx), _ptr(dweight), _ptr(dbias),
                          _ptr(d_init), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    if rc:
        raise KdaError("kda_conv_bwd", rc)
    return dx, dweight, dbias, d_init


def conv_decode(x, weight, state_pool, bias=None, state_indices=None, num_commit=None, silu=False, out=None,
                out_dtype=None):
    """Decode / replay step of the convolution: x [B, T, D]; state_pool float32 [P, W-1, D] updated in place;
    state_indices / num_commit int32 [B] as for decode().  Returns y [B, T, D] (out_dtype, default float32)."""
    import torch
    lib = load_library()
    dev = x.device
    W = _conv_params(weight, bias, x.shape[-1], dev)
    desc, (B, T, D, _), odt = _conv_desc(x, W, None, out_dtype, silu, decode=True)
    if state_pool.dim() != 3:
        raise ValueError("state_pool must be [P, W-1, D]")
    _check("state_pool", state_pool, torch.float32, (state_pool.shape[0], W - 1, D), dev)
    for name, t in (("state_indices", state_indices), ("num_commit", num_commit)):
        if t is not None:
            _check(name, t, torch.int32, (B,), dev)
    if out is None:
        out = torch.empty((B, T, D), dtype=odt, device=dev)
    else:
        _check("out", out, odt, (B, T, D), dev)
    rc = lib.kda_conv_decode(ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(bias), _ptr(state_pool),
                             int(state_pool.shape[0]), _ptr(state_indices), _ptr(num_commit), _ptr(out),
                             _stream(dev))
    if rc:
        raise KdaError("kda_conv_decode", rc)
    return out
