"""ctypes binding of the C ABI in include/ssm_scan.h.

Argument marshalling only: checks that tensors live on the current HIP device
with the dtype and layout the ABI documents, allocates outputs and workspace
with torch, and passes raw device pointers plus torch's current stream to the
library. Every arithmetic step runs in the library's HIP kernels; there is no
fallback. A missing library, a CPU tensor or a non-zero status raises.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSM_SCAN_LIBRARY names another build of the same ABI (the test suite's
# sanitizer build of the host-side front end, whose launches always fail).
LIB_PATH = os.environ.get("SSM_SCAN_LIBRARY") or os.path.join(_HERE, "lib", "libssm_scan.so")

SSM_F32, SSM_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: SSM_F32, torch.bfloat16: SSM_BF16}

_lib = None
_lock = threading.Lock()


class SSMError(RuntimeError):
    """Non-zero status from the library."""

    def __init__(self, fn, status, message):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not found at {LIB_PATH}; build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        lib.ssm_abi_version.restype = i32
        lib.ssm_abi_version.argtypes = []
        lib.ssm_status_string.restype = ctypes.c_char_p
        lib.ssm_status_string.argtypes = [i32]
        lib.ssm_scan_workspace_bytes.restype = sz
        lib.ssm_scan_workspace_bytes.argtypes = [i64, i64, i64, i64]
        lib.ssm_scan_chunks.restype = i64
        lib.ssm_scan_chunks.argtypes = [i64, i64, i64, i64]
        lib.ssm_selective_scan_fwd.restype = i32
        lib.ssm_selective_scan_fwd.argtypes = [i64, i64, i64, i64, i32, i32, i32,
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, sz, vp]
        lib.ssm_selective_scan_fwd_noalloc.restype = i32
        lib.ssm_selective_scan_fwd_noalloc.argtypes = [i64, i64, i64, i64, i32, i32, i32,
                                                       vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                       vp, vp, vp]
        lib.ssm_selective_state_update.restype = i32
        lib.ssm_selective_state_update.argtypes = [i64, i64, i64, i32, i32, i32,
                                                   vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                   vp, vp]
        lib.ssm_scan_bwd_workspace_bytes.restype = sz
        lib.ssm_scan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
        lib.ssm_selective_scan_bwd.restype = i32
        lib.ssm_selective_scan_bwd.argtypes = [i64, i64, i64, i64, i32, i32] + [vp] * 21 + [sz, vp]
        lib.ssm_scan_checkpoint_bytes.restype = sz
        lib.ssm_scan_checkpoint_bytes.argtypes = [i64, i64, i64, i64]
        lib.ssm_selective_scan_fwd_ckpt.restype = i32
        lib.ssm_selective_scan_fwd_ckpt.argtypes = [i64, i64, i64, i64, i32, i32, i32] + [vp] * 13 + [sz, vp]
        lib.ssm_selective_scan_bwd_ckpt.restype = i32
        lib.ssm_selective_scan_bwd_ckpt.argtypes = [i64, i64, i64, i64, i32, i32] + [vp] * 22 + [sz, vp]
        lib.ssm_causal_conv1d_fwd.restype = i32
        lib.ssm_causal_conv1d_fwd.argtypes = [i64, i64, i64, i64, i32, i32, i32,
                                              vp, vp, vp, vp, vp, vp, vp]
        lib.ssm_causal_conv1d_update.restype = i32
        lib.ssm_causal_conv1d_update.argtypes = [i64, i64, i64, i32, i32, i32,
                                                 vp, vp, vp, vp, vp, vp]
        lib.ssm_ssd_fwd.restype = i32
        lib.ssm_ssd_fwd.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32] + [vp] * 11 + [vp]
        _lib = lib
        return lib


def library():
    """The loaded ctypes library (loads it on first call)."""
    return _load()


def _check(fn, status):
    if status != 0:
        msg = _load().ssm_status_string(status).decode()
        raise SSMError(fn, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(name, t, shape, dtypes, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")
    return t


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _launch_context(device, stream):
    """The device current, and the stream the kernels are enqueued on current
    too: what the binding allocates here (outputs, workspace) is then owned by
    that stream in torch's caching allocator, so a workspace dropped after the
    call is not handed to work on another stream while the kernels still use it."""
    ctx = contextlib.ExitStack()
    ctx.enter_context(torch.cuda.device(device))
    if stream is not None:
        ctx.enter_context(torch.cuda.stream(stream))
    return ctx


def _check_workspace(workspace, dev):
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace.numel() * workspace.element_size()


def ssm_abi_version() -> int:
    return int(_load().ssm_abi_version())


def ssm_scan_workspace_bytes(batch, seqlen, dim, dstate) -> int:
    return int(_load().ssm_scan_workspace_bytes(batch, seqlen, dim, dstate))


FLAG_SOFTPLUS = 1   # SSM_FLAG_SOFTPLUS
FLAG_ZOH = 2        # SSM_FLAG_ZOH


def _flags(delta_softplus, zoh):
    return (FLAG_SOFTPLUS if delta_softplus else 0) | (FLAG_ZOH if zoh else 0)


def ssm_scan_chunks(batch, seqlen, dim, dstate) -> int:
    """Sequence chunks the scan of this shape runs in (1 = single pass, 0 = unsupported)."""
    return int(_load().ssm_scan_chunks(batch, seqlen, dim, dstate))


def ssm_selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                           delta_softplus=False, h0=None, out_dtype=None,
                           return_final_state=False, y=None, h_final=None,
                           workspace=None, stream=None, zoh=False, checkpoints=None):
    """Selective scan forward; see ssm_selective_scan_fwd in include/ssm_scan.h.

    u, delta, z: [B, L, d]; B, C: [B, L, N] (all float32 or all bfloat16);
    A: [d, N], D, delta_bias: [d], h0: [B, d, N] (float32).
    ``zoh`` selects the exact zero-order-hold input coefficient (SSM_FLAG_ZOH).
    ``checkpoints``: a float32 tensor of ssm_scan_checkpoint_bytes() bytes, or
    True to allocate one: calls ssm_selective_scan_fwd_ckpt, which also writes
    the backward's state checkpoints there (N <= 16).
    Returns y ([B, L, d], ``out_dtype`` or the input dtype) or (y, h_final);
    with checkpoints, (y, h_final, checkpoints).
    """
    lib = _load()
    if not isinstance(u, torch.Tensor) or u.dim() != 3:
        raise ValueError("u must be a 3-d tensor [B, L, d]")
    dev = u.device
    Bt, L, d = u.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a 2-d tensor [d, N]")
    N = A.shape[1]
    ind = (u.dtype,)
    if u.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {u.dtype}")
    _dev_tensor("u", u, (Bt, L, d), ind, dev)
    _dev_tensor("delta", delta, (Bt, L, d), ind, dev)
    _dev_tensor("A", A, (d, N), (torch.float32,), dev)
    _dev_tensor("B", B, (Bt, L, N), ind, dev)
    _dev_tensor("C", C, (Bt, L, N), ind, dev)
    _dev_tensor("D", D, (d,), (torch.float32,), dev)
    _dev_tensor("z", z, (Bt, L, d), ind, dev)
    _dev_tensor("delta_bias", delta_bias, (d,), (torch.float32,), dev)
    _dev_tensor("h0", h0, (Bt, d, N), (torch.float32,), dev)
    out_dtype = u.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    with _launch_context(dev, stream):
        if y is None:
            y = torch.empty((Bt, L, d), dtype=out_dtype, device=dev)
        _dev_tensor("y", y, (Bt, L, d), (out_dtype,), dev)
        if return_final_state and h_final is None:
            h_final = torch.empty((Bt, d, N), dtype=torch.float32, device=dev)
        _dev_tensor("h_final", h_final, (Bt, d, N), (torch.float32,), dev)
        ws_bytes = int(lib.ssm_scan_workspace_bytes(Bt, L, d, N))
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        ws_size = _check_workspace(workspace, dev)
        if checkpoints is None:
            st = lib.ssm_selective_scan_fwd(
                Bt, L, d, N, _DTYPE_CODE[u.dtype], _DTYPE_CODE[out_dtype], _flags(delta_softplus, zoh),
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                _ptr(h0), _ptr(y), _ptr(h_final), _ptr(workspace), ws_size, _stream_handle(stream, dev))
        else:
            ck_bytes = int(lib.ssm_scan_checkpoint_bytes(Bt, L, d, N))
            if checkpoints is True:
                checkpoints = torch.empty(max(ck_bytes // 4, 1), dtype=torch.float32, device=dev)
            _check_checkpoints(checkpoints, ck_bytes, dev)
            st = lib.ssm_selective_scan_fwd_ckpt(
                Bt, L, d, N, _DTYPE_CODE[u.dtype], _DTYPE_CODE[out_dtype], _flags(delta_softplus, zoh),
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                _ptr(h0), _ptr(y), _ptr(h_final), _ptr(checkpoints), _ptr(workspace), ws_size,
                _stream_handle(stream, dev))
    _check("ssm_selective_scan_fwd" + ("" if checkpoints is None else "_ckpt"), st)
    if checkpoints is not None:
        return y, h_final, checkpoints
    if return_final_state or h_final is not None:
        return y, h_final
    return y


def ssm_selective_scan_fwd_noalloc(u, delta, A, B, C, y, D=None, z=None, delta_bias=None,
                                   delta_softplus=False, h0=None, h_final=None, stream=None, zoh=False):
    """Selective scan forward with the library's own scratch array as its
    workspace; see ssm_selective_scan_fwd_noalloc in include/ssm_scan.h.

    Arguments as ssm_selective_scan_fwd, except that the output y (and h_final,
    when wanted) must be given: nothing is allocated on this path. Returns y,
    or (y, h_final).
    """
    lib = _load()
    if not isinstance(u, torch.Tensor) or u.dim() != 3 or u.dtype not in _DTYPE_CODE:
        raise ValueError("u must be a 3-d float32 or bfloat16 tensor [B, L, d]")
    dev = u.device
    Bt, L, d = u.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a 2-d tensor [d, N]")
    N = A.shape[1]
    ind = (u.dtype,)
    _dev_tensor("u", u, (Bt, L, d), ind, dev)
    _dev_tensor("delta", delta, (Bt, L, d), ind, dev)
    _dev_tensor("A", A, (d, N), (torch.float32,), dev)
    _dev_tensor("B", B, (Bt, L, N), ind, dev)
    _dev_tensor("C", C, (Bt, L, N), ind, dev)
    _dev_tensor("D", D, (d,), (torch.float32,), dev)
    _dev_tensor("z", z, (Bt, L, d), ind, dev)
    _dev_tensor("delta_bias", delta_bias, (d,), (torch.float32,), dev)
    _dev_tensor("h0", h0, (Bt, d, N), (torch.float32,), dev)
    if not isinstance(y, torch.Tensor) or y.dtype not in _DTYPE_CODE:
        raise ValueError("y must be a float32 or bfloat16 tensor [B, L, d]")
    _dev_tensor("y", y, (Bt, L, d), (y.dtype,), dev)
    _dev_tensor("h_final", h_final, (Bt, d, N), (torch.float32,), dev)
    with torch.cuda.device(dev):
        st = lib.ssm_selective_scan_fwd_noalloc(
            Bt, L, d, N, _DTYPE_CODE[u.dtype], _DTYPE_CODE[y.dtype], _flags(delta_softplus, zoh),
            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            _ptr(h0), _ptr(y), _ptr(h_final), _stream_handle(stream, dev))
    _check("ssm_selective_scan_fwd_noalloc", st)
    return y if h_final is None else (y, h_final)


def ssm_selective_state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                               delta_softplus=False, out_dtype=None, y=None, stream=None, zoh=False):
    """One decode step in place on ``state``; see ssm_selective_state_update in include/ssm_scan.h.

    state: [B, d, N] float32 (updated in place); x, delta, z: [B, d]; B, C: [B, N]
    (all float32 or all bfloat16); A: [d, N], D, delta_bias: [d] float32.
    ``zoh`` as in ssm_selective_scan_fwd. Returns y [B, d].
    """
    lib = _load()
    if not isinstance(state, torch.Tensor) or state.dim() != 3:
        raise ValueError("state must be a 3-d tensor [B, d, N]")
    dev = state.device
    Bt, d, N = state.shape
    if not isinstance(x, torch.Tensor) or x.dtype not in _DTYPE_CODE:
        raise ValueError("x must be a float32 or bfloat16 tensor")
    ind = (x.dtype,)
    _dev_tensor("state", state, (Bt, d, N), (torch.float32,), dev)
    _dev_tensor("x", x, (Bt, d), ind, dev)
    _dev_tensor("delta", delta, (Bt, d), ind, dev)
    _dev_tensor("A", A, (d, N), (torch.float32,), dev)
    _dev_tensor("B", B, (Bt, N), ind, dev)
    _dev_tensor("C", C, (Bt, N), ind, dev)
    _dev_tensor("D", D, (d,), (torch.float32,), dev)
    _dev_tensor("z", z, (Bt, d), ind, dev)
    _dev_tensor("delta_bias", delta_bias, (d,), (torch.float32,), dev)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    with _launch_context(dev, stream):
        if y is None:
            y = torch.empty((Bt, d), dtype=out_dtype, device=dev)
        _dev_tensor("y", y, (Bt, d), (out_dtype,), dev)
        st = lib.ssm_selective_state_update(
            Bt, d, N, _DTYPE_CODE[x.dtype], _DTYPE_CODE[out_dtype], _flags(delta_softplus, zoh),
            _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), _ptr(y), _stream_handle(stream, dev))
    _check("ssm_selective_state_update", st)
    return y


def ssm_causal_conv1d_fwd(x, weight, bias=None, state_in=None, silu_activation=True, out_dtype=None,
                          return_final_state=False, y=None, state_out=None, stream=None):
    """Causal depthwise conv1d (+ SiLU); see ssm_causal_conv1d_fwd in include/ssm_scan.h.

    x: [B, L, d] float32 or bfloat16; weight: [d, K], bias: [d], state_in: [B, d, K-1]
    (float32). Returns y ([B, L, d]) or (y, state_out).
    """
    lib = _load()
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a 3-d tensor [B, L, d]")
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    dev = x.device
    Bt, L, d = x.shape
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a 2-d tensor [d, K]")
    K = weight.shape[1]
    _dev_tensor("x", x, (Bt, L, d), (x.dtype,), dev)
    _dev_tensor("weight", weight, (d, K), (torch.float32,), dev)
    _dev_tensor("bias", bias, (d,), (torch.float32,), dev)
    _dev_tensor("state_in", state_in, (Bt, d, K - 1), (torch.float32,), dev)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    with _launch_context(dev, stream):
        if y is None:
            y = torch.empty((Bt, L, d), dtype=out_dtype, device=dev)
        _dev_tensor("y", y, (Bt, L, d), (out_dtype,), dev)
        if return_final_state and state_out is None:
            state_out = torch.empty((Bt, d, K - 1), dtype=torch.float32, device=dev)
        _dev_tensor("state_out", state_out, (Bt, d, K - 1), (torch.float32,), dev)
        st = lib.ssm_causal_conv1d_fwd(Bt, L, d, K, _DTYPE_CODE[x.dtype], _DTYPE_CODE[out_dtype],
                                       int(bool(silu_activation)), _ptr(x), _ptr(weight), _ptr(bias),
                                       _ptr(state_in), _ptr(y), _ptr(state_out), _stream_handle(stream, dev))
    _check("ssm_causal_conv1d_fwd", st)
    if return_final_state or state_out is not None:
        return y, state_out
    return y


def ssm_causal_conv1d_update(state, x, weight, bias=None, silu_activation=True, out_dtype=None,
                             y=None, stream=None):
    """One token through the convolution, state updated in place; see
    ssm_causal_conv1d_update in include/ssm_scan.h.

    state: [B, d, K-1] float32 (in place); x: [B, d]; weight: [d, K], bias: [d].
    Returns y [B, d].
    """
    lib = _load()
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.dtype not in _DTYPE_CODE:
        raise ValueError("x must be a 2-d float32 or bfloat16 tensor [B, d]")
    dev = x.device
    Bt, d = x.shape
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a 2-d tensor [d, K]")
    K = weight.shape[1]
    _dev_tensor("x", x, (Bt, d), (x.dtype,), dev)
    _dev_tensor("weight", weight, (d, K), (torch.float32,), dev)
    _dev_tensor("bias", bias, (d,), (torch.float32,), dev)
    if K > 1 or state is not None:
        _dev_tensor("state", state, (Bt, d, K - 1), (torch.float32,), dev)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    with _launch_context(dev, stream):
        if y is None:
            y = torch.empty((Bt, d), dtype=out_dtype, device=dev)
        _dev_tensor("y", y, (Bt, d), (out_dtype,), dev)
        st = lib.ssm_causal_conv1d_update(Bt, d, K, _DTYPE_CODE[x.dtype], _DTYPE_CODE[out_dtype],
                                          int(bool(silu_activation)), _ptr(state), _ptr(x), _ptr(weight),
                                          _ptr(bias), _ptr(y), _stream_handle(stream, dev))
    _check("ssm_causal_conv1d_update", st)
    return y


def ssm_scan_checkpoint_bytes(batch, seqlen, dim, dstate) -> int:
    return int(_load().ssm_scan_checkpoint_bytes(batch, seqlen, dim, dstate))


def _check_checkpoints(ck, need, dev):
    if not isinstance(ck, torch.Tensor) or ck.dtype != torch.float32 or ck.device != dev or not ck.is_contiguous():
        raise ValueError("checkpoints must be a contiguous float32 tensor on the inputs' device")
    if ck.numel() * 4 < need:
        raise ValueError(f"checkpoints hold {ck.numel() * 4} bytes, {need} needed")


def ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate) -> int:
    return int(_load().ssm_scan_bwd_workspace_bytes(batch, seqlen, dim, dstate))


def ssm_selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False,
                           h0=None, dh_final=None, workspace=None, stream=None, zoh=False, checkpoints=None):
    """Gradients of the selective scan; see ssm_selective_scan_bwd in include/ssm_scan.h.

    Inputs as ssm_selective_scan_fwd, plus dy [B, L, d] and dh_final [B, d, N]
    (float32). Returns a dict of float32 tensors: du, ddelta, dA, dB, dC, dh0,
    and dD / dz / ddelta_bias when D / z / delta_bias are given. ``zoh``: the
    gradients of the exact zero-order-hold forward (SSM_FLAG_ZOH).
    ``checkpoints``: the tensor ssm_selective_scan_fwd(..., checkpoints=...)
    filled for the same inputs and h0: calls ssm_selective_scan_bwd_ckpt.
    """
    lib = _load()
    if not isinstance(u, torch.Tensor) or u.dim() != 3 or u.dtype not in _DTYPE_CODE:
        raise ValueError("u must be a 3-d float32 or bfloat16 tensor [B, L, d]")
    dev = u.device
    Bt, L, d = u.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a 2-d tensor [d, N]")
    N = A.shape[1]
    ind = (u.dtype,)
    f32 = (torch.float32,)
    _dev_tensor("u", u, (Bt, L, d), ind, dev)
    _dev_tensor("delta", delta, (Bt, L, d), ind, dev)
    _dev_tensor("A", A, (d, N), f32, dev)
    _dev_tensor("B", B, (Bt, L, N), ind, dev)
    _dev_tensor("C", C, (Bt, L, N), ind, dev)
    _dev_tensor("D", D, (d,), f32, dev)
    _dev_tensor("z", z, (Bt, L, d), ind, dev)
    _dev_tensor("delta_bias", delta_bias, (d,), f32, dev)
    _dev_tensor("h0", h0, (Bt, d, N), f32, dev)
    _dev_tensor("dy", dy, (Bt, L, d), f32, dev)
    _dev_tensor("dh_final", dh_final, (Bt, d, N), f32, dev)
    new = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)  # noqa: E731
    with _launch_context(dev, stream):
        g = dict(du=new(Bt, L, d), ddelta=new(Bt, L, d), dA=new(d, N), dB=new(Bt, L, N), dC=new(Bt, L, N),
                 dh0=new(Bt, d, N))
        if D is not None:
            g["dD"] = new(d)
        if z is not None:
            g["dz"] = new(Bt, L, d)
        if delta_bias is not None:
            g["ddelta_bias"] = new(d)
        ws_bytes = int(lib.ssm_scan_bwd_workspace_bytes(Bt, L, d, N))
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        ws_size = _check_workspace(workspace, dev)
        args = [Bt, L, d, N, _DTYPE_CODE[u.dtype], _flags(delta_softplus, zoh),
                _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0),
                _ptr(dy), _ptr(dh_final), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")), _ptr(g["dh0"])]
        if checkpoints is None:
            st = lib.ssm_selective_scan_bwd(*args, _ptr(workspace), ws_size, _stream_handle(stream, dev))
        else:
            _check_checkpoints(checkpoints, int(lib.ssm_scan_checkpoint_bytes(Bt, L, d, N)), dev)
            st = lib.ssm_selective_scan_bwd_ckpt(*args, _ptr(checkpoints), _ptr(workspace), ws_size,
                                                 _stream_handle(stream, dev))
    _check("ssm_selective_scan_bwd" + ("" if checkpoints is None else "_ckpt"), st)
    return g


def ssm_ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, h0=None, out_dtype=None,
                return_final_state=False, y=None, h_final=None, stream=None):
    """Mamba-2 SSD layer forward; see ssm_ssd_fwd in include/ssm_scan.h.

    x, z: [B, L, H, P]; dt: [B, L, H]; B, C: [B, L, N] (all float32 or all
    bfloat16); A, D, dt_bias: [H] float32; h0: [B, H, P, N] float32.
    Returns y ([B, L, H, P]) or (y, h_final).
    """
    lib = _load()
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a 4-d tensor [B, L, H, P]")
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    dev = x.device
    Bt, L, H, P = x.shape
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise ValueError("B must be a 3-d tensor [B, L, N]")
    N = B.shape[2]
    ind = (x.dtype,)
    _dev_tensor("x", x, (Bt, L, H, P), ind, dev)
    _dev_tensor("dt", dt, (Bt, L, H), ind, dev)
    _dev_tensor("A", A, (H,), (torch.float32,), dev)
    _dev_tensor("B", B, (Bt, L, N), ind, dev)
    _dev_tensor("C", C, (Bt, L, N), ind, dev)
    _dev_tensor("D", D, (H,), (torch.float32,), dev)
    _dev_tensor("z", z, (Bt, L, H, P), ind, dev)
    _dev_tensor("dt_bias", dt_bias, (H,), (torch.float32,), dev)
    _dev_tensor("h0", h0, (Bt, H, P, N), (torch.float32,), dev)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    with _launch_context(dev, stream):
        if y is None:
            y = torch.empty((Bt, L, H, P), dtype=out_dtype, device=dev)
        _dev_tensor("y", y, (Bt, L, H, P), (out_dtype,), dev)
        if return_final_state and h_final is None:
            h_final = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
        _dev_tensor("h_final", h_final, (Bt, H, P, N), (torch.float32,), dev)
        st = lib.ssm_ssd_fwd(Bt, L, H, P, N, _DTYPE_CODE[x.dtype], _DTYPE_CODE[out_dtype],
                             _flags(dt_softplus, False), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final), _stream_handle(stream, dev))
    _check("ssm_ssd_fwd", st)
    if return_final_state or h_final is not None:
        return y, h_final
    return y
