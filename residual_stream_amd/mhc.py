"""Python binding of the mHC C ABI (include/mhc.h): argument marshalling only.

Every step of hc_pre / hc_post and their backward runs in the gfx950 kernels of
``libmhc.so``; this module turns torch tensors into device pointers, allocates
outputs and workspaces with torch (the library itself never allocates), and
passes torch's current HIP stream.  There is no fallback: if the library is
missing or the tensors are not on the GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmhc.so")

MHC_F32 = 0
MHC_BF16 = 1
MHC_OK = 0
MHC_ERR_INVALID_ARG = 1
MHC_ERR_UNSUPPORTED = 2
MHC_ERR_HIP = 3
MHC_ERR_TOO_LARGE = 4

ABI_FUNCTIONS = (
    "mhc_pre_workspace_bytes",
    "mhc_pre",
    "mhc_post",
    "mhc_post_bwd",
    "mhc_pre_bwd_workspace_bytes",
    "mhc_pre_bwd",
    "mhc_pre_bwd_mix",
    "mhc_post_pre_workspace_bytes",
    "mhc_post_pre",
    "mhc_post_stable",
    "mhc_post_stable_bwd_workspace_bytes",
    "mhc_post_stable_bwd",
    "mhc_pre_noalloc",
    "mhc_status_string",
    "mhc_abi_version",
    "mhc_trace_kernel_events",
    "mhc_test_exchange_fault",
)


class MhcDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("N", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("io", ctypes.c_int32),
        ("sinkhorn_iters", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("alpha_pre", ctypes.c_float),
        ("alpha_post", ctypes.c_float),
        ("alpha_res", ctypes.c_float),
        ("alpha", ctypes.c_void_p),
    ]


class MhcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


_lib = None
_P = ctypes.c_void_p
_DP = ctypes.POINTER(MhcDesc)


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmhc.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m residual_stream_amd.build`")
    lib = ctypes.CDLL(p)
    lib.mhc_abi_version.restype = ctypes.c_int
    lib.mhc_abi_version.argtypes = []
    lib.mhc_status_string.restype = ctypes.c_char_p
    lib.mhc_status_string.argtypes = [ctypes.c_int]
    for name in ("mhc_pre_workspace_bytes", "mhc_pre_bwd_workspace_bytes", "mhc_post_pre_workspace_bytes"):
        f = getattr(lib, name)
        f.restype = ctypes.c_size_t
        f.argtypes = [_DP]
    lib.mhc_pre.restype = ctypes.c_int
    lib.mhc_pre.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_post.restype = ctypes.c_int
    lib.mhc_post.argtypes = [_DP, _P, _P, _P, _P, _P, _P]
    lib.mhc_post_bwd.restype = ctypes.c_int
    lib.mhc_post_bwd.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.mhc_pre_bwd.restype = ctypes.c_int
    lib.mhc_pre_bwd.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_pre_bwd_mix.restype = ctypes.c_int
    lib.mhc_pre_bwd_mix.argtypes = [_DP] + [_P] * 13 + [ctypes.c_size_t, _P]
    lib.mhc_post_pre.restype = ctypes.c_int
    lib.mhc_post_pre.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mhc_post_stable.restype = ctypes.c_int
    lib.mhc_post_stable.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.mhc_post_stable_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.mhc_post_stable_bwd_workspace_bytes.argtypes = [_DP, ctypes.c_int, ctypes.c_int]
    lib.mhc_post_stable_bwd.restype = ctypes.c_int
    lib.mhc_post_stable_bwd.argtypes = [_DP] + [_P] * 14 + [ctypes.c_size_t, _P]
    lib.mhc_pre_noalloc.restype = ctypes.c_int
    lib.mhc_pre_noalloc.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.mhc_trace_kernel_events.restype = ctypes.c_int
    lib.mhc_trace_kernel_events.argtypes = [_P, _P, ctypes.c_int, _P]
    lib.mhc_test_exchange_fault.restype = ctypes.c_int
    lib.mhc_test_exchange_fault.argtypes = [ctypes.c_int, ctypes.c_uint]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mhc_status_string(int(status)).decode()


def make_desc(T: int, N: int, D: int, io: int, iters: int = 20, eps: float = 1e-6,
              alphas=(0.01, 0.01, 0.01)) -> MhcDesc:
    """Descriptor of one call.  `alphas` is three floats (pre, post, res), or a
    float32 GPU tensor of at least three elements that the kernels read on the
    device (a trained α: no host round trip, and graph replays follow it)."""
    if isinstance(alphas, torch.Tensor):
        if not alphas.is_cuda or alphas.dtype != torch.float32 or alphas.numel() < 3 or not alphas.is_contiguous():
            raise ValueError("a device alpha must be a contiguous float32 GPU tensor of 3 elements")
        return MhcDesc(int(T), int(N), int(D), int(io), int(iters), float(eps), 0.0, 0.0, 0.0,
                       alphas.data_ptr())
    a = tuple(alphas)
    return MhcDesc(int(T), int(N), int(D), int(io), int(iters), float(eps), float(a[0]),
                   float(a[1]), float(a[2]), None)


def _io_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MHC_F32
    if t.dtype == torch.bfloat16:
        return MHC_BF16
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise RuntimeError("the mHC kernels need GPU tensors (no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != MHC_OK:
        raise MhcError(status, where)


def _f32(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.float32:
        raise TypeError(f"{tuple(t.shape)} tensor must be float32")
    return t


def _workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace for one call (contents on entry are ignored by the library)."""
    if torch.device(device).type != "cuda":
        raise RuntimeError("the mHC kernels need GPU tensors (no CPU path)")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_bytes(ws) -> int:
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("a workspace must be a contiguous GPU tensor")
    return ws.numel() * ws.element_size()


def _expect(name, t, shape, dtype, device, optional=False):
    """Shape, dtype, device and layout of one tensor argument, checked before
    any pointer reaches the C ABI (which cannot check sizes itself)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:  # (device is x's, a GPU: host tensors are refused here)
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _state(x):
    """(T, N, D, io dtype, device) of a state tensor x[T, N, D]."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [T, N, D] tensor")
    _io_of(x)
    if not x.is_cuda:
        raise RuntimeError("the mHC kernels need GPU tensors (no CPU path)")
    if x.device.index != torch.cuda.current_device():
        raise ValueError(f"x is on {x.device}; make it the current device first")
    T, N, D = x.shape
    return T, N, D, x.dtype, x.device


def _coef_shapes(T, N, D):
    return {"x": (T, N, D), "y": (T, D), "phi": (N * D, N * N + 2 * N), "bias": (N * N + 2 * N,),
            "H": (T, N), "H_res": (T, N, N)}


def desc_for(x: torch.Tensor, iters: int = 20, eps: float = 1e-6, alphas=(0.01, 0.01, 0.01)):
    T, N, D = x.shape
    return make_desc(T, N, D, _io_of(x), iters, eps, alphas)


def mhc_pre(x, phi, bias, *, iters=20, eps=1e-6, alphas=(0.01, 0.01, 0.01), out=None,
            workspace=None, stream=None):
    """hc_pre forward.  x[T,N,D] (fp32/bf16), phi[N·D,C], bias[C] fp32.

    Returns (h[T,D], H_pre[T,N], H_post[T,N], H_res[T,N,N])."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, iters, eps, alphas)
    sh = _coef_shapes(T, N, D)
    _expect("phi", phi, sh["phi"], torch.float32, dv)
    _expect("bias", bias, sh["bias"], torch.float32, dv)
    if out is None:
        out = (torch.empty((T, D), dtype=x.dtype, device=x.device),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N, N), dtype=torch.float32, device=x.device))
    h, Hp, Hq, Hr = out
    _expect("h", h, (T, D), io, dv)
    _expect("H_pre", Hp, sh["H"], torch.float32, dv)
    _expect("H_post", Hq, sh["H"], torch.float32, dv)
    _expect("H_res", Hr, sh["H_res"], torch.float32, dv)
    need = lib.mhc_pre_workspace_bytes(ctypes.byref(d))
    if workspace is None and need:
        workspace = _workspace(need, x.device)
    nbytes = _ws_bytes(workspace)
    st = lib.mhc_pre(ctypes.byref(d), _ptr(x), _ptr(_f32(phi)), _ptr(_f32(bias)), _ptr(h), _ptr(Hp),
                     _ptr(Hq), _ptr(Hr), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "mhc_pre")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20  # MHC_NOALLOC_SCRATCH_BYTES of include/mhc.h


def mhc_pre_noalloc(x, phi, bias, *, iters=20, eps=1e-6, alphas=(0.01, 0.01, 0.01), out=None, stream=None):
    """hc_pre on the library's static scratch buffer (``mhc_pre_noalloc``):
    no workspace, and with ``out`` given no allocation at all.  Results equal
    :func:`mhc_pre`'s bit for bit; raises MhcError with status
    MHC_ERR_TOO_LARGE where the call needs more than the buffer holds.  Calls
    that overlap in time on one GPU race on its buffer.

    Returns (h[T,D], H_pre[T,N], H_post[T,N], H_res[T,N,N])."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, iters, eps, alphas)
    sh = _coef_shapes(T, N, D)
    _expect("phi", phi, sh["phi"], torch.float32, dv)
    _expect("bias", bias, sh["bias"], torch.float32, dv)
    if out is None:
        out = (torch.empty((T, D), dtype=x.dtype, device=x.device),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N, N), dtype=torch.float32, device=x.device))
    h, Hp, Hq, Hr = out
    _expect("h", h, (T, D), io, dv)
    _expect("H_pre", Hp, sh["H"], torch.float32, dv)
    _expect("H_post", Hq, sh["H"], torch.float32, dv)
    _expect("H_res", Hr, sh["H_res"], torch.float32, dv)
    st = lib.mhc_pre_noalloc(ctypes.byref(d), _ptr(x), _ptr(_f32(phi)), _ptr(_f32(bias)), _ptr(h), _ptr(Hp),
                             _ptr(Hq), _ptr(Hr), _stream(stream))
    _check(st, "mhc_pre_noalloc")
    return out


def mhc_post(x, y, H_post, H_res, *, out=None, stream=None):
    """hc_post forward: returns x_next[T,N,D] in x's dtype."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x)
    sh = _coef_shapes(T, N, D)
    _expect("y", y, sh["y"], io, dv)
    _expect("H_post", H_post, sh["H"], torch.float32, dv)
    _expect("H_res", H_res, sh["H_res"], torch.float32, dv)
    if out is None:
        out = torch.empty_like(x)
    _expect("x_next", out, sh["x"], io, dv)
    st = lib.mhc_post(ctypes.byref(d), _ptr(x), _ptr(y), _ptr(_f32(H_post)), _ptr(_f32(H_res)),
                      _ptr(out), _stream(stream))
    _check(st, "mhc_post")
    return out


def mhc_post_bwd(dx_next, x, y, H_post, H_res, *, want_dx=True, out=None, stream=None):
    """hc_post backward: returns (dx[T,N,D], dy[T,D], dH_post[T,N], dH_res[T,N,N]).
    With want_dx=False (or a None dx in `out`) dx is not formed (None is
    returned in its place): :func:`mhc_pre_bwd_mix` forms it from dx_next."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x)
    sh = _coef_shapes(T, N, D)
    _expect("dx_next", dx_next, sh["x"], io, dv)
    _expect("y", y, sh["y"], io, dv)
    _expect("H_post", H_post, sh["H"], torch.float32, dv)
    _expect("H_res", H_res, sh["H_res"], torch.float32, dv)
    if out is None:
        out = (torch.empty_like(x) if want_dx else None, torch.empty_like(y),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N, N), dtype=torch.float32, device=x.device))
    dx, dy, dHp, dHr = out
    _expect("dx", dx, sh["x"], io, dv, optional=True)
    _expect("dy", dy, sh["y"], io, dv)
    _expect("dH_post", dHp, sh["H"], torch.float32, dv)
    _expect("dH_res", dHr, sh["H_res"], torch.float32, dv)
    st = lib.mhc_post_bwd(ctypes.byref(d), _ptr(dx_next), _ptr(x), _ptr(y), _ptr(_f32(H_post)),
                          _ptr(_f32(H_res)), _ptr(dx), _ptr(dy), _ptr(dHp), _ptr(dHr),
                          _stream(stream))
    _check(st, "mhc_post_bwd")
    return out


def mhc_pre_bwd(dh, x, phi, bias, dH_post, dH_res, dx, *, iters=20, eps=1e-6,
                alphas=(0.01, 0.01, 0.01), want_dalpha=True, out=None, workspace=None,
                stream=None):
    """hc_pre backward with recompute.  `dx` holds hc_post's contribution on
    entry and the total on return (updated in place).

    Returns (dx, dphi[K,C], dbias[C], dalpha[3] or None)."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, iters, eps, alphas)
    C = N * N + 2 * N
    sh = _coef_shapes(T, N, D)
    _expect("dh", dh, sh["y"], io, dv)
    _expect("phi", phi, sh["phi"], torch.float32, dv)
    _expect("bias", bias, sh["bias"], torch.float32, dv)
    _expect("dH_post", dH_post, sh["H"], torch.float32, dv)
    _expect("dH_res", dH_res, sh["H_res"], torch.float32, dv)
    _expect("dx", dx, sh["x"], io, dv)
    if out is None:
        out = (torch.empty((N * D, C), dtype=torch.float32, device=x.device),
               torch.empty((C,), dtype=torch.float32, device=x.device),
               torch.empty((4,), dtype=torch.float32, device=x.device) if want_dalpha else None)
    dphi, dbias, dalpha = out
    _check_grad_outs(dphi, dbias, dalpha, sh, dv)
    need = lib.mhc_pre_bwd_workspace_bytes(ctypes.byref(d))
    if workspace is None and need:
        workspace = _workspace(need, x.device)
    nbytes = _ws_bytes(workspace)
    st = lib.mhc_pre_bwd(ctypes.byref(d), _ptr(dh), _ptr(x), _ptr(_f32(phi)), _ptr(_f32(bias)),
                         _ptr(_f32(dH_post)), _ptr(_f32(dH_res)), _ptr(dx), _ptr(dphi),
                         _ptr(dbias), _ptr(dalpha), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "mhc_pre_bwd")
    return dx, dphi, dbias, (dalpha[:3] if dalpha is not None else None)


def _check_grad_outs(dphi, dbias, dalpha, sh, dv):
    _expect("dphi", dphi, sh["phi"], torch.float32, dv)
    _expect("dbias", dbias, sh["bias"], torch.float32, dv)
    if dalpha is not None:
        if not isinstance(dalpha, torch.Tensor) or not dalpha.is_cuda or dalpha.dtype != torch.float32 \
                or dalpha.numel() < 3 or not dalpha.is_contiguous() or dalpha.device != dv:
            raise ValueError("dalpha must be a contiguous float32 GPU tensor of at least 3 elements")


def mix_fuses(N: int, D: int, io: int, iters: int = 20) -> bool:
    """True where mhc_pre_bwd_mix forms H_resᵀ·dx_next inside the hc_pre
    backward's dx pass (bf16, N = 4, D a multiple of 256: the matrix-core
    path), so that the pair mhc_post_bwd(want_dx=False) + mhc_pre_bwd_mix moves
    a state-sized tensor less than mhc_post_bwd + mhc_pre_bwd.  Elsewhere the
    library runs the mix as a kernel of its own first, and the two calls are
    the faster choice (the results are the same bits either way)."""
    return io == MHC_BF16 and N == 4 and D % 256 == 0 and iters <= 64


def mhc_pre_bwd_mix(dh, x, phi, bias, dH_post, dH_res, dx_next, H_res, *, iters=20, eps=1e-6,
                    alphas=(0.01, 0.01, 0.01), want_dalpha=True, out=None, workspace=None, stream=None):
    """hc_pre backward with hc_post's share of the state gradient formed
    inside it: dx = H_resᵀ·dx_next + the hc_pre part (pair with
    ``mhc_post_bwd(..., want_dx=False)``).

    Returns (dx[T,N,D], dphi[K,C], dbias[C], dalpha[3] or None)."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, iters, eps, alphas)
    C = N * N + 2 * N
    sh = _coef_shapes(T, N, D)
    _expect("dh", dh, sh["y"], io, dv)
    _expect("phi", phi, sh["phi"], torch.float32, dv)
    _expect("bias", bias, sh["bias"], torch.float32, dv)
    _expect("dH_post", dH_post, sh["H"], torch.float32, dv)
    _expect("dH_res", dH_res, sh["H_res"], torch.float32, dv)
    _expect("dx_next", dx_next, sh["x"], io, dv)
    _expect("H_res", H_res, sh["H_res"], torch.float32, dv)
    if out is None:
        out = (torch.empty_like(x), torch.empty((N * D, C), dtype=torch.float32, device=x.device),
               torch.empty((C,), dtype=torch.float32, device=x.device),
               torch.empty((4,), dtype=torch.float32, device=x.device) if want_dalpha else None)
    dx, dphi, dbias, dalpha = out
    _expect("dx", dx, sh["x"], io, dv)
    _check_grad_outs(dphi, dbias, dalpha, sh, dv)
    need = lib.mhc_pre_bwd_workspace_bytes(ctypes.byref(d))
    if workspace is None and need:
        workspace = _workspace(need, x.device)
    nbytes = _ws_bytes(workspace)
    st = lib.mhc_pre_bwd_mix(ctypes.byref(d), _ptr(dh), _ptr(x), _ptr(_f32(phi)), _ptr(_f32(bias)),
                             _ptr(_f32(dH_post)), _ptr(_f32(dH_res)), _ptr(dx_next), _ptr(_f32(H_res)),
                             _ptr(dx), _ptr(dphi), _ptr(dbias), _ptr(dalpha), _ptr(workspace), nbytes,
                             _stream(stream))
    _check(st, "mhc_pre_bwd_mix")
    return dx, dphi, dbias, (dalpha[:3] if dalpha is not None else None)


def mhc_post_pre(x, y, H_post, H_res, phi, bias, *, iters=20, eps=1e-6, alphas=(0.01, 0.01, 0.01),
                 out=None, workspace=None, stream=None):
    """hc_post of one layer fused with hc_pre of the next: x_next = H_res·x +
    H_post ⊗ y, then hc_pre(x_next; phi, bias) of the next layer.

    Returns (x_next[T,N,D], h[T,D], H_pre[T,N], H_post[T,N], H_res[T,N,N])."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, iters, eps, alphas)
    sh = _coef_shapes(T, N, D)
    _expect("y", y, sh["y"], io, dv)
    _expect("H_post", H_post, sh["H"], torch.float32, dv)
    _expect("H_res", H_res, sh["H_res"], torch.float32, dv)
    _expect("phi", phi, sh["phi"], torch.float32, dv)
    _expect("bias", bias, sh["bias"], torch.float32, dv)
    if out is None:
        out = (torch.empty_like(x), torch.empty((T, D), dtype=x.dtype, device=x.device),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N), dtype=torch.float32, device=x.device),
               torch.empty((T, N, N), dtype=torch.float32, device=x.device))
    xn, h, Hp, Hq, Hr = out
    for name, t, shape, dt in (("x_next", xn, sh["x"], io), ("h", h, sh["y"], io), ("H_pre out", Hp, sh["H"], torch.float32),
                               ("H_post out", Hq, sh["H"], torch.float32), ("H_res out", Hr, sh["H_res"], torch.float32)):
        _expect(name, t, shape, dt, dv)
    need = lib.mhc_post_pre_workspace_bytes(ctypes.byref(d))
    if workspace is None and need:
        workspace = _workspace(need, x.device)
    nbytes = _ws_bytes(workspace)
    st = lib.mhc_post_pre(ctypes.byref(d), _ptr(x), _ptr(y), _ptr(_f32(H_post)), _ptr(_f32(H_res)),
                          _ptr(_f32(phi)), _ptr(_f32(bias)), _ptr(xn), _ptr(h), _ptr(Hp), _ptr(Hq),
                          _ptr(Hr), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "mhc_post_pre")
    return out


def workspace_bytes(kind: str, T: int, N: int, D: int, io: int, iters: int = 20, *,
                    y_weight: bool = False, out_weight: bool = False) -> int:
    """Workspace size (host-only query) for 'pre', 'pre_bwd', 'post_pre' or
    'post_stable_bwd' (with the given norm weights present)."""
    lib = load()
    d = make_desc(T, N, D, io, iters)
    if kind == "post_stable_bwd":
        return int(lib.mhc_post_stable_bwd_workspace_bytes(ctypes.byref(d), int(y_weight), int(out_weight)))
    f = {"pre": lib.mhc_pre_workspace_bytes, "pre_bwd": lib.mhc_pre_bwd_workspace_bytes,
         "post_pre": lib.mhc_post_pre_workspace_bytes}[kind]
    return int(f(ctypes.byref(d)))


def mhc_post_stable(x, y, H_post, H_res, *, y_weight=None, out_weight=None, eps=1e-6, out=None,
                    stream=None):
    """Stabilised write-back: sandwich norm of y (weight y_weight[D]) before
    H_post writes it back and block post-norm of the state (weight
    out_weight[N·D]) after; either weight may be None.  Returns x_next."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, eps=eps)
    sh = _coef_shapes(T, N, D)
    _expect("y", y, sh["y"], io, dv)
    _expect("H_post", H_post, sh["H"], torch.float32, dv)
    _expect("H_res", H_res, sh["H_res"], torch.float32, dv)
    _expect("y_weight", y_weight, (D,), torch.float32, dv, optional=True)
    _expect("out_weight", out_weight, (N * D,), torch.float32, dv, optional=True)
    if out is None:
        out = torch.empty_like(x)
    _expect("x_next", out, sh["x"], io, dv)
    yw = None if y_weight is None else _f32(y_weight)
    ow = None if out_weight is None else _f32(out_weight)
    st = lib.mhc_post_stable(ctypes.byref(d), _ptr(x), _ptr(y), _ptr(yw), _ptr(_f32(H_post)),
                             _ptr(_f32(H_res)), _ptr(ow), _ptr(out), _stream(stream))
    _check(st, "mhc_post_stable")
    return out


def mhc_post_stable_bwd(dx_next, x, y, H_post, H_res, *, y_weight=None, out_weight=None, eps=1e-6,
                        out=None, workspace=None, stream=None):
    """Backward of :func:`mhc_post_stable`.  Returns (dx, dy, dH_post, dH_res,
    dy_weight or None, dout_weight or None)."""
    lib = load()
    T, N, D, io, dv = _state(x)
    d = desc_for(x, eps=eps)
    sh = _coef_shapes(T, N, D)
    sw, pn = y_weight is not None, out_weight is not None
    _expect("dx_next", dx_next, sh["x"], io, dv)
    _expect("y", y, sh["y"], io, dv)
    _expect("H_post", H_post, sh["H"], torch.float32, dv)
    _expect("H_res", H_res, sh["H_res"], torch.float32, dv)
    _expect("y_weight", y_weight, (D,), torch.float32, dv, optional=True)
    _expect("out_weight", out_weight, (N * D,), torch.float32, dv, optional=True)
    if out is None:
        f32 = dict(dtype=torch.float32, device=x.device)
        out = (torch.empty_like(x), torch.empty_like(y), torch.empty((T, N), **f32),
               torch.empty((T, N, N), **f32), torch.empty(D, **f32) if sw else None,
               torch.empty(N * D, **f32) if pn else None)
    dx, dy, dHp, dHr, dyw, dow = out
    _expect("dx", dx, sh["x"], io, dv)
    _expect("dy", dy, sh["y"], io, dv)
    _expect("dH_post", dHp, sh["H"], torch.float32, dv)
    _expect("dH_res", dHr, sh["H_res"], torch.float32, dv)
    _expect("dy_weight", dyw, (D,), torch.float32, dv, optional=not sw)
    _expect("dout_weight", dow, (N * D,), torch.float32, dv, optional=not pn)
    need = lib.mhc_post_stable_bwd_workspace_bytes(ctypes.byref(d), int(sw), int(pn))
    if workspace is None and need:
        workspace = _workspace(need, x.device)
    nbytes = _ws_bytes(workspace)
    st = lib.mhc_post_stable_bwd(
        ctypes.byref(d), _ptr(dx_next), _ptr(x), _ptr(y),
        _ptr(None if y_weight is None else _f32(y_weight)), _ptr(_f32(H_post)), _ptr(_f32(H_res)),
        _ptr(None if out_weight is None else _f32(out_weight)), _ptr(dx), _ptr(dy), _ptr(dyw),
        _ptr(dow), _ptr(dHp), _ptr(dHr), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "mhc_post_stable_bwd")
    return out


class KernelTrace:
    """Kernel-level HIP-event timing of the library's launches on this host
    thread (``mhc_trace_kernel_events``): use as a context manager around the
    calls to time, then read :meth:`durations_us` after synchronising.  The
    events are torch's, recorded by the library on each call's stream."""

    def __init__(self, capacity: int = 64):
        self.capacity = int(capacity)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * self.capacity)]
        cur = torch.cuda.current_stream()
        for e in self.events:  # creates the underlying HIP events
            e.record(cur)
        self._handles = (ctypes.c_void_p * (2 * self.capacity))(*[e.cuda_event for e in self.events])
        self._names = (ctypes.c_char_p * self.capacity)()
        self._count = ctypes.c_int(0)

    def __enter__(self):
        _check(load().mhc_trace_kernel_events(self._handles, self._names, self.capacity,
                                              ctypes.byref(self._count)), "mhc_trace_kernel_events")
        return self

    def __exit__(self, *exc):
        load().mhc_trace_kernel_events(None, None, 0, None)
        return False

    def durations_us(self):
        """[(kernel name, µs)] of the launches recorded (synchronise first)."""
        n = self._count.value
        return [(self._names[k].decode(), self.events[2 * k].elapsed_time(self.events[2 * k + 1]) * 1e3)
                for k in range(n)]
