"""Thin Python binding of libmesa (include/mesa.h): argument marshalling only.

Every step of the Mesa layer runs in the library's HIP kernels; this module
allocates outputs with torch, passes raw device pointers and the current HIP
stream, and maps status codes to Python exceptions.  There is no fallback:
if libmesa.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmesa.so")

MESA_OK, MESA_ERR_INVALID_ARGUMENT, MESA_ERR_UNSUPPORTED, MESA_ERR_WORKSPACE_TOO_SMALL, MESA_ERR_HIP = range(5)
MESA_DTYPE_F32, MESA_DTYPE_BF16 = 0, 1
KERNEL_CHUNK_STATES, KERNEL_CG_OUTPUT, KERNEL_DECODE, KERNEL_QK_PREPROCESS = 0, 1, 2, 3
KERNEL_BWD_ADJOINT, KERNEL_BWD_STATES, KERNEL_BWD_KV, KERNEL_BWD_GATE, KERNEL_HAWK = 4, 5, 6, 7, 8
MESA_WARM_COLD, MESA_WARM_PREVIOUS, MESA_WARM_PROJECTED = 0, 1, 2

# Every symbol include/mesa.h declares, with its ctypes signature.
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "mesa_abi_version": ([], _I),
    "mesa_status_string": ([_I], ctypes.c_char_p),
    "mesa_last_error_message": ([], ctypes.c_char_p),
    "mesa_forward_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _Z),
    "mesa_forward": ([_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                      _P, _P, _P, _P, _P, _Z, _P], _I),
    "mesa_forward_train": ([_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                            _P, _P, _P, _P, _Z, _P], _I),
    "mesa_forward_noalloc": ([_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                              _P, _P, _P, _P, _P], _I),
    "mesa_backward_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _Z),
    "mesa_backward": ([_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                       _P, _P, _P, _P, _P, _P, _P, _Z, _P], _I),
    "mesa_decode_step": ([_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F,
                          _P, _P, _P], _I),
    "mesa_decode_step_warm": ([_P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                               _P, _P, _P], _I),
    "mesa_qk_preprocess": ([_P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _P, _I, _P], _I),
    "mesa_hawk_workspace_bytes": ([_I, _I, _I], _Z),
    "mesa_hawk_scan": ([_P, _P, _P, _I, _P, _F, _P, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "mesa_profile_enable": ([_I], _I),
    "mesa_profile_read": ([_I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)], _I),
    "mesa_profile_reset": ([], _I),
    "mesa_kernel_name": ([_I], ctypes.c_char_p),
    # include/mesa_probe.h
    "mesa_probe_mfma_f32": ([_I, _I, _P, _P], _I),
    "mesa_probe_mfma_bf16": ([_I, _I, _P, _P], _I),
    "mesa_probe_copy": ([_P, _P, _Z, _P], _I),
}

_lib = None


class MesaError(RuntimeError):
    """A HIP runtime failure reported by libmesa."""


def lib():
    """The loaded libmesa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status == MESA_OK:
        return
    L = lib()
    msg = f"{what}: {L.mesa_status_string(status).decode()}: {L.mesa_last_error_message().decode()}"
    if status in (MESA_ERR_INVALID_ARGUMENT, MESA_ERR_WORKSPACE_TOO_SMALL):
        raise ValueError(msg)
    if status == MESA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise MesaError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _qkv_dtype(t):
    import torch
    if t.dtype == torch.float32:
        return MESA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MESA_DTYPE_BF16
    raise ValueError(f"q/k/v dtype {t.dtype} is not float32 or bfloat16")


def _need(t, name, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dims(t, name, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {list(t.shape)}")
    return tuple(t.shape)


def _shapes(*specs):
    """Every (tensor, name, shape) must have exactly that shape.  Checked
    before any device or dtype check, so that a mis-shaped argument is named
    whatever else is wrong."""
    for t, name, shape in specs:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _shape(t, name, shape, dtype=None, device=None):
    """A device tensor of exactly this shape (and dtype/device, when given)."""
    _shapes((t, name, shape))
    _need(t, name, dtype, device)


def _given(*specs):
    """The (tensor, name, shape) specs whose tensor was given."""
    return tuple(sp for sp in specs if sp[0] is not None)


def _forward_checks(q, k, v, gamma, lam, **outs):
    """Shapes, dtypes and devices of mesa_forward's inputs, and the shapes of
    the outputs the caller passed (out, iters, x_out, final_H, final_G);
    returns (B, H, T, dk, dv)."""
    import torch
    B, H, T, dk = _dims(q, "q", 4)
    dv = _dims(v, "v", 4)[-1]
    oshape = dict(out=(B, H, T, dv), iters=(B, H, T), x_out=(B, H, T, dk), final_H=(B, H, dk, dk),
                  final_G=(B, H, dv, dk))
    _shapes((k, "k", (B, H, T, dk)), (v, "v", (B, H, T, dv)), (gamma, "gamma", (B, H, T)),
            (lam, "lambda", (H, dk)), *_given(*((t, n, oshape[n]) for n, t in outs.items())))
    _qkv_dtype(q)
    for t, n, dt in ((q, "q", q.dtype), (k, "k", q.dtype), (v, "v", q.dtype), (gamma, "gamma", torch.float32),
                     (lam, "lambda", torch.float32)):
        _need(t, n, dt, q.device)
    return B, H, T, dk, dv


def _out(t, name, shape, dtype, device):
    """A caller-provided output: checked like an input, or allocated."""
    import torch
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _shape(t, name, shape, dtype, device)
    return t


def mesa_forward_workspace_bytes(B, H, T, dk, dv, chunk) -> int:
    return int(lib().mesa_forward_workspace_bytes(B, H, T, dk, dv, chunk))


def mesa_forward(q, k, v, gamma, lam, max_iters, tol=0.0, chunk=64, *, out=None, iters=None,
                 return_iters=True, return_final=False, final_H=None, final_G=None,
                 workspace=None, stream=None):
    """Mesa-layer forward (see include/mesa.h, mesa_forward).

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (float32 or bfloat16, same dtype);
    gamma: [B,H,T] float32; lam: [H,dk] float32.  Returns (out, iters,
    final_H, final_G); iters/final_* are None unless requested.
    """
    import torch
    B, H, T, dk, dv = _forward_checks(q, k, v, gamma, lam, out=out, iters=iters, final_H=final_H,
                                      final_G=final_G)
    dev = q.device
    dt = _qkv_dtype(q)
    out = _out(out, "out", (B, H, T, dv), torch.float32, dev)
    if iters is not None or return_iters:
        iters = _out(iters, "iters", (B, H, T), torch.int32, dev)
    if return_final or final_H is not None or final_G is not None:
        final_H = _out(final_H, "final_H", (B, H, dk, dk), torch.float32, dev)
        final_G = _out(final_G, "final_G", (B, H, dv, dk), torch.float32, dev)
    ws_bytes = mesa_forward_workspace_bytes(B, H, T, dk, dv, chunk) if max_iters > 0 else 0
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", None, dev)
    st = lib().mesa_forward(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(gamma), _ptr(lam),
                            B, H, T, dk, dv, int(chunk), int(max_iters), float(tol),
                            _ptr(out), _ptr(iters), _ptr(final_H), _ptr(final_G),
                            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check(st, "mesa_forward")
    return out, iters, final_H, final_G


def mesa_forward_noalloc(q, k, v, gamma, lam, max_iters, tol=0.0, chunk=64, *, out, iters=None, final_H=None,
                         final_G=None, stream=None):
    """mesa_forward with the chunk states in the library's built-in device
    array (see include/mesa.h, mesa_forward_noalloc): the caller passes every
    output, and the call allocates nothing.  Returns (out, iters, final_H,
    final_G) as given."""
    B, H, T, dk, dv = _forward_checks(q, k, v, gamma, lam, out=out, iters=iters, final_H=final_H,
                                      final_G=final_G)
    import torch
    dev = q.device
    _need(out, "out", torch.float32, dev)
    for t, n, dt in ((iters, "iters", torch.int32), (final_H, "final_H", torch.float32),
                     (final_G, "final_G", torch.float32)):
        if t is not None:
            _need(t, n, dt, dev)
    st = lib().mesa_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _qkv_dtype(q), _ptr(gamma), _ptr(lam),
                                    B, H, T, dk, dv, int(chunk), int(max_iters), float(tol),
                                    _ptr(out), _ptr(iters), _ptr(final_H), _ptr(final_G), _stream(stream))
    _check(st, "mesa_forward_noalloc")
    return out, iters, final_H, final_G


def mesa_forward_train(q, k, v, gamma, lam, max_iters, tol=0.0, chunk=64, *, out=None, iters=None,
                       x_out=None, workspace=None, stream=None):
    """Forward that also returns the CG solutions x (see include/mesa.h,
    mesa_forward_train).  Returns (out, iters, x)."""
    import torch
    B, H, T, dk, dv = _forward_checks(q, k, v, gamma, lam, out=out, iters=iters, x_out=x_out)
    dev = q.device
    out = _out(out, "out", (B, H, T, dv), torch.float32, dev)
    iters = _out(iters, "iters", (B, H, T), torch.int32, dev)
    x_out = _out(x_out, "x_out", (B, H, T, dk), torch.float32, dev)
    nbytes = mesa_forward_workspace_bytes(B, H, T, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    st = lib().mesa_forward_train(_ptr(q), _ptr(k), _ptr(v), _qkv_dtype(q), _ptr(gamma), _ptr(lam),
                                  B, H, T, dk, dv, chunk, int(max_iters), float(tol),
                                  _ptr(out), _ptr(iters), _ptr(x_out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    _check(st, "mesa_forward_train")
    return out, iters, x_out


def mesa_backward_workspace_bytes(B, H, T, dk, dv, chunk) -> int:
    return int(lib().mesa_backward_workspace_bytes(B, H, T, dk, dv, chunk))


def mesa_backward(k, v, gamma, lam, x, out, grad_out, max_iters, tol=0.0, chunk=64, *, workspace=None,
                  return_z_iters=True, stream=None):
    """Backward pass (see include/mesa.h, mesa_backward).  Returns a dict of
    grad_q, grad_k, grad_v, grad_gamma, grad_lambda (float32) and z_iters."""
    import torch
    B, H, T, dk = _dims(k, "k", 4)
    dv = _dims(v, "v", 4)[-1]
    dev = k.device
    _shapes((v, "v", (B, H, T, dv)), (gamma, "gamma", (B, H, T)), (lam, "lambda", (H, dk)),
            (x, "x", (B, H, T, dk)), (out, "out", (B, H, T, dv)), (grad_out, "grad_out", (B, H, T, dv)))
    _qkv_dtype(k)
    for t, n, dt in ((k, "k", k.dtype), (v, "v", k.dtype), (gamma, "gamma", torch.float32),
                     (lam, "lambda", torch.float32), (x, "x", torch.float32), (out, "out", torch.float32),
                     (grad_out, "grad_out", torch.float32)):
        _need(t, n, dt, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(grad_q=torch.empty((B, H, T, dk), **f32), grad_k=torch.empty((B, H, T, dk), **f32),
             grad_v=torch.empty((B, H, T, dv), **f32), grad_gamma=torch.empty((B, H, T), **f32),
             grad_lambda=torch.empty((H, dk), **f32))
    g["z_iters"] = torch.empty((B, H, T), dtype=torch.int32, device=dev) if return_z_iters else None
    nbytes = mesa_backward_workspace_bytes(B, H, T, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    st = lib().mesa_backward(_ptr(k), _ptr(v), _qkv_dtype(k), _ptr(gamma), _ptr(lam), _ptr(x), _ptr(out),
                             _ptr(grad_out), B, H, T, dk, dv, chunk, int(max_iters), float(tol),
                             _ptr(g["grad_q"]), _ptr(g["grad_k"]), _ptr(g["grad_v"]), _ptr(g["grad_gamma"]),
                             _ptr(g["grad_lambda"]), _ptr(g["z_iters"]), _ptr(workspace),
                             workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check(st, "mesa_backward")
    return g


def _decode_checks(q, k, v, gamma, lam, state_H, state_G, state_x=None, out=None, iters=None):
    import torch
    N, H, dk = _dims(q, "q", 3)
    dv = _dims(v, "v", 3)[-1]
    dev = q.device
    specs = [(k, "k", (N, H, dk)), (v, "v", (N, H, dv)), (gamma, "gamma", (N, H)), (lam, "lambda", (H, dk)),
             (state_H, "state_H", (N, H, dk, dk)), (state_G, "state_G", (N, H, dv, dk)),
             *_given((out, "out", (N, H, dv)), (iters, "iters", (N, H)))]
    if state_x is not None:
        specs.append((state_x, "state_x", (N, H, dk)))
    _shapes(*specs)
    _qkv_dtype(q)
    for t, n, dt in ((q, "q", q.dtype), (k, "k", q.dtype), (v, "v", q.dtype), (gamma, "gamma", torch.float32),
                     (lam, "lambda", torch.float32), (state_H, "state_H", torch.float32),
                     (state_G, "state_G", torch.float32)):
        _need(t, n, dt, dev)
    if state_x is not None:
        _need(state_x, "state_x", torch.float32, dev)
    return N, H, dk, dv, dev


def mesa_decode_step(q, k, v, gamma, lam, state_H, state_G, max_iters, tol=0.0, *,
                     out=None, iters=None, return_iters=True, stream=None):
    """One decode step (see include/mesa.h, mesa_decode_step); state_H/G updated in place.

    q, k: [N,H,dk]; v: [N,H,dv]; gamma: [N,H]; lam: [H,dk];
    state_H: [N,H,dk,dk], state_G: [N,H,dv,dk] float32.  Returns (out, iters).
    """
    import torch
    N, H, dk, dv, dev = _decode_checks(q, k, v, gamma, lam, state_H, state_G, out=out, iters=iters)
    out = _out(out, "out", (N, H, dv), torch.float32, dev)
    if iters is not None or return_iters:
        iters = _out(iters, "iters", (N, H), torch.int32, dev)
    st = lib().mesa_decode_step(_ptr(q), _ptr(k), _ptr(v), _qkv_dtype(q), _ptr(gamma), _ptr(lam),
                                _ptr(state_H), _ptr(state_G), N, H, dk, dv, int(max_iters),
                                float(tol), _ptr(out), _ptr(iters), _stream(stream))
    _check(st, "mesa_decode_step")
    return out, iters


def mesa_decode_step_warm(q, k, v, gamma, lam, state_H, state_G, state_x, max_iters, tol=0.0,
                          warm_mode=MESA_WARM_PROJECTED, *, out=None, iters=None, return_iters=True,
                          stream=None):
    """One warm-started decode step (see include/mesa.h, mesa_decode_step_warm).

    As mesa_decode_step, plus state_x [N,H,dk] float32: the previous
    solutions on entry, this step's on exit.  Returns (out, iters).
    """
    import torch
    N, H, dk, dv, dev = _decode_checks(q, k, v, gamma, lam, state_H, state_G, state_x, out=out, iters=iters)
    out = _out(out, "out", (N, H, dv), torch.float32, dev)
    if iters is not None or return_iters:
        iters = _out(iters, "iters", (N, H), torch.int32, dev)
    st = lib().mesa_decode_step_warm(_ptr(q), _ptr(k), _ptr(v), _qkv_dtype(q), _ptr(gamma), _ptr(lam),
                                     _ptr(state_H), _ptr(state_G), _ptr(state_x), N, H, dk, dv,
                                     int(max_iters), float(tol), int(warm_mode), _ptr(out), _ptr(iters),
                                     _stream(stream))
    _check(st, "mesa_decode_step_warm")
    return out, iters


def mesa_qk_preprocess(x, conv_w, hist=None, *, out_dtype=None, out=None, return_hist=False,
                       hist_out=None, stream=None):
    """Causal convolution of width W over tokens + L2 normalisation (see include/mesa.h).

    x: [B,H,T,d] float32 or bfloat16; conv_w: [H,W,d] float32; hist: [B,H,W-1,d]
    in x's dtype or None.  Returns y (out_dtype, default x's dtype), and with
    return_hist also hist_out, the last W-1 input rows for the next piece.
    """
    import torch
    B, H, T, d = _dims(x, "x", 4)
    W = _dims(conv_w, "conv_w", 3)[1]
    dev = x.device
    _shapes((conv_w, "conv_w", (H, W, d)), *(((hist, "hist", (B, H, W - 1, d)),) if hist is not None else ()))
    _qkv_dtype(x)
    _need(x, "x", None, dev)
    _need(conv_w, "conv_w", torch.float32, dev)
    if hist is not None:
        _need(hist, "hist", x.dtype, dev)
    out_dtype = (x.dtype if out is None else out.dtype) if out_dtype is None else out_dtype
    out = _out(out, "out", (B, H, T, d), out_dtype, dev)
    if return_hist or hist_out is not None:
        hist_out = _out(hist_out, "hist_out", (B, H, W - 1, d), x.dtype, dev)
    st = lib().mesa_qk_preprocess(_ptr(x), _qkv_dtype(x), _ptr(conv_w), W, _ptr(hist), _ptr(hist_out),
                                  B, H, T, d, _ptr(out), _qkv_dtype(out), _stream(stream))
    _check(st, "mesa_qk_preprocess")
    return (out, hist_out) if return_hist else out


def mesa_hawk_scan(x, ga, gx, lam, c=8.0, h0=None, *, out=None, return_final=False, workspace=None,
                   stream=None):
    """The Hawk layer's gated linear recurrence (see include/mesa.h, mesa_hawk_scan).

    x, ga, gx: [B,T,D] float32 or bfloat16 (same dtype); lam: [D] float32;
    h0: [B,D] float32 or None.  Returns y [B,T,D] float32 (and h_final [B,D]).
    """
    import torch
    B, T, D = _dims(x, "x", 3)
    dev = x.device
    _shapes((ga, "ga", (B, T, D)), (gx, "gx", (B, T, D)), (lam, "lam", (D,)),
            *(((h0, "h0", (B, D)),) if h0 is not None else ()))
    _qkv_dtype(x)
    for t, n, dt in ((x, "x", x.dtype), (ga, "ga", x.dtype), (gx, "gx", x.dtype), (lam, "lam", torch.float32)):
        _need(t, n, dt, dev)
    if h0 is not None:
        _need(h0, "h0", torch.float32, dev)
    out = _out(out, "out", (B, T, D), torch.float32, dev)
    hf = torch.empty((B, D), dtype=torch.float32, device=dev) if return_final else None
    nbytes = int(lib().mesa_hawk_workspace_bytes(B, T, D))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, dev)
    st = lib().mesa_hawk_scan(_ptr(x), _ptr(ga), _ptr(gx), _qkv_dtype(x), _ptr(lam), float(c), _ptr(h0), B, T, D,
                              _ptr(out), _ptr(hf), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream))
    _check(st, "mesa_hawk_scan")
    return (out, hf) if return_final else out


def profile_enable(on: bool = True):
    _check(lib().mesa_profile_enable(1 if on else 0), "mesa_profile_enable")


def profile_reset():
    _check(lib().mesa_profile_reset(), "mesa_profile_reset")


def profile_read(kernel_id: int):
    """(total milliseconds, launches) recorded for one kernel id since the last reset."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(lib().mesa_profile_read(kernel_id, ctypes.byref(ms), ctypes.byref(n)), "mesa_profile_read")
    return ms.value, n.value


def probe_mfma(dtype: str, n_workgroups: int, iters: int, sink, stream=None):
    """Launch the register-resident MFMA probe ("f32" or "bf16"); returns its flops."""
    fn = lib().mesa_probe_mfma_f32 if dtype == "f32" else lib().mesa_probe_mfma_bf16
    _check(fn(n_workgroups, iters, _ptr(sink), _stream(stream)), "mesa_probe_mfma")
    return n_workgroups * 4 * iters * 8 * (2048 if dtype == "f32" else 16384)


def probe_copy(src, dst, stream=None):
    """Launch the streaming-copy probe over src.numel() bytes of src (uint8) into dst."""
    _check(lib().mesa_probe_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(), _stream(stream)),
           "mesa_probe_copy")


def kernel_name(kernel_id: int) -> str:
    return lib().mesa_kernel_name(kernel_id).decode()
