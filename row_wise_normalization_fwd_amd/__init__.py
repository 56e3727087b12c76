"""Row-wise RMSNorm (and LayerNorm) for MI355X (gfx950): Python binding of
librmsnorm_mi355x.so.

The C ABI (include/rmsnorm_mi355x.h) is exposed under the same names
(``rmsnorm_fwd``, ``rmsnorm_fused_add_fwd``, ``rmsnorm_bwd``,
``rmsnorm_fused_add_bwd``, ``rmsnorm_bwd_noalloc``, ``rmsnorm_quant_fwd``, ``rmsnorm_qk_fwd``,
``layernorm_fwd``,
``layernorm_bwd``, ``layernorm_bwd_workspace_size``, ``rmsnorm_bwd_workspace_size``,
``rmsnorm_status_string``,
``rmsnorm_last_hip_error``); those functions only marshal arguments. Pointers
may be given as integers or as torch tensors (their ``data_ptr()``); streams as
integers or ``torch.cuda.Stream`` objects.

``fwd``, ``fused_add_fwd``, ``quant_fwd``, ``qk_fwd``, ``bwd``, ``fused_add_bwd``,
``layernorm`` and ``layernorm_backward`` are torch conveniences on top: they use
torch only to allocate outputs and to pick the current stream, and every step
of the computation runs in the library's HIP kernels. There is no fallback: if
the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "librmsnorm_mi355x.so"
LIB_PATH = os.path.join(_HERE, LIB_NAME)

RMSN_F32, RMSN_F16, RMSN_BF16 = 0, 1, 2
RMSN_QUANT_FP8_TENSOR, RMSN_QUANT_FP8_ROW, RMSN_QUANT_MXFP8, RMSN_QUANT_MXFP4 = 1, 2, 3, 4
RMSN_OK = 0
STATUS_NAMES = {
    0: "RMSN_OK", -1: "RMSN_ERR_NULL", -2: "RMSN_ERR_SHAPE", -3: "RMSN_ERR_DTYPE",
    -4: "RMSN_ERR_WORKSPACE", -5: "RMSN_ERR_OVERLAP", -6: "RMSN_ERR_ALIGN",
    -7: "RMSN_ERR_EPS", -8: "RMSN_ERR_MODE", -9: "RMSN_ERR_SCRATCH", -100: "RMSN_ERR_HIP",
}
RMSN_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
ENTRY_POINTS = ("rmsnorm_fwd", "rmsnorm_fused_add_fwd", "rmsnorm_quant_fwd", "rmsnorm_qk_fwd",
                "layernorm_fwd", "layernorm_bwd", "layernorm_bwd_workspace_size", "rmsnorm_bwd",
                "rmsnorm_fused_add_bwd", "rmsnorm_bwd_workspace_size", "rmsnorm_bwd_noalloc",
                "rmsnorm_status_string", "rmsnorm_last_hip_error")


class RMSNormError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        msg = f"{where} failed: {name}: {rmsnorm_status_string(status)}"
        if status == -100:
            msg += f" (hipError {rmsnorm_last_hip_error()})"
        super().__init__(msg)


_lib = None


def load_library(path: str | None = None):
    """Load the built HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{LIB_NAME} is not built at {path}; build it with "
            "`python -m row_wise_normalization_fwd_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.rmsnorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_fwd.restype = i32
    lib.rmsnorm_fused_add_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_fused_add_fwd.restype = i32
    lib.rmsnorm_quant_fwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_quant_fwd.restype = i32
    lib.rmsnorm_qk_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32, i32,
                                   vp]
    lib.rmsnorm_qk_fwd.restype = i32
    lib.layernorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.layernorm_fwd.restype = i32
    lib.layernorm_bwd_workspace_size.argtypes = [i64, i64]
    lib.layernorm_bwd_workspace_size.restype = ctypes.c_size_t
    lib.layernorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64,
                                  i32, i32, vp]
    lib.layernorm_bwd.restype = i32
    lib.rmsnorm_bwd_workspace_size.argtypes = [i64, i64]
    lib.rmsnorm_bwd_workspace_size.restype = ctypes.c_size_t
    lib.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i32, i32, vp]
    lib.rmsnorm_bwd.restype = i32
    lib.rmsnorm_fused_add_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64,
                                          i32, i32, vp]
    lib.rmsnorm_fused_add_bwd.restype = i32
    lib.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, vp]
    lib.rmsnorm_bwd_noalloc.restype = i32
    lib.rmsnorm_status_string.argtypes = [i32]
    lib.rmsnorm_status_string.restype = ctypes.c_char_p
    lib.rmsnorm_last_hip_error.argtypes = []
    lib.rmsnorm_last_hip_error.restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _p(v):
    """Pointer argument: None, an int address, or a device tensor's
    data_ptr(). A host tensor is refused: its address would reach the GPU."""
    if v is None:
        return None
    if isinstance(v, int):
        return v or None
    if getattr(v, "is_cuda", True) is False:
        raise ValueError(f"a host tensor ({v.device}) was passed where device memory is required")
    return v.data_ptr() or None


def _s(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


# ------------------------------------------------------- C ABI, same names

def rmsnorm_fwd(x, gamma, y, rstd, M, N, eps, x_dtype, gamma_dtype, stream) -> int:
    return load_library().rmsnorm_fwd(_p(x), _p(gamma), _p(y), _p(rstd), M, N, eps,
                                      x_dtype, gamma_dtype, _s(stream))


def rmsnorm_fused_add_fwd(x, residual, gamma, y, rstd, M, N, eps, x_dtype, gamma_dtype,
                          stream) -> int:
    return load_library().rmsnorm_fused_add_fwd(_p(x), _p(residual), _p(gamma), _p(y), _p(rstd),
                                                M, N, eps, x_dtype, gamma_dtype, _s(stream))


def rmsnorm_quant_fwd(x, residual, gamma, q, scale, quant_mode, rstd, M, N, eps, x_dtype,
                      gamma_dtype, stream) -> int:
    return load_library().rmsnorm_quant_fwd(_p(x), _p(residual), _p(gamma), _p(q), _p(scale),
                                            quant_mode, _p(rstd), M, N, eps, x_dtype,
                                            gamma_dtype, _s(stream))


def rmsnorm_qk_fwd(q, k, q_gamma, k_gamma, tokens, q_heads, k_heads, head_dim, q_stride,
                   k_stride, eps, x_dtype, gamma_dtype, stream) -> int:
    return load_library().rmsnorm_qk_fwd(_p(q), _p(k), _p(q_gamma), _p(k_gamma), tokens, q_heads,
                                         k_heads, head_dim, q_stride, k_stride, eps, x_dtype,
                                         gamma_dtype, _s(stream))


def layernorm_fwd(x, gamma, beta, y, mean, rstd, M, N, eps, x_dtype, gamma_dtype, stream) -> int:
    return load_library().layernorm_fwd(_p(x), _p(gamma), _p(beta), _p(y), _p(mean), _p(rstd), M,
                                        N, eps, x_dtype, gamma_dtype, _s(stream))


def layernorm_bwd_workspace_size(M, N) -> int:
    return int(load_library().layernorm_bwd_workspace_size(M, N))


def layernorm_bwd(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, workspace, workspace_bytes, M, N,
                  x_dtype, gamma_dtype, stream) -> int:
    return load_library().layernorm_bwd(_p(dy), _p(x), _p(mean), _p(rstd), _p(gamma), _p(dx),
                                        _p(dgamma), _p(dbeta), _p(workspace), workspace_bytes, M,
                                        N, x_dtype, gamma_dtype, _s(stream))


def rmsnorm_bwd_workspace_size(M, N) -> int:
    return int(load_library().rmsnorm_bwd_workspace_size(M, N))


def rmsnorm_bwd(dy, x, rstd, gamma, dx, dgamma, workspace, workspace_bytes, M, N, x_dtype,
                gamma_dtype, stream) -> int:
    return load_library().rmsnorm_bwd(_p(dy), _p(x), _p(rstd), _p(gamma), _p(dx), _p(dgamma),
                                      _p(workspace), workspace_bytes, M, N, x_dtype, gamma_dtype,
                                      _s(stream))


def rmsnorm_bwd_noalloc(dy, x, rstd, gamma, dx, dgamma, M, N, x_dtype, gamma_dtype,
                        stream) -> int:
    return load_library().rmsnorm_bwd_noalloc(_p(dy), _p(x), _p(rstd), _p(gamma), _p(dx),
                                              _p(dgamma), M, N, x_dtype, gamma_dtype, _s(stream))


def rmsnorm_fused_add_bwd(dy, h, rstd, gamma, dresidual, dh, dgamma, workspace, workspace_bytes,
                          M, N, x_dtype, gamma_dtype, stream) -> int:
    return load_library().rmsnorm_fused_add_bwd(_p(dy), _p(h), _p(rstd), _p(gamma),
                                                _p(dresidual), _p(dh), _p(dgamma), _p(workspace),
                                                workspace_bytes, M, N, x_dtype, gamma_dtype,
                                                _s(stream))


def rmsnorm_status_string(status: int) -> str:
    return load_library().rmsnorm_status_string(status).decode()


def rmsnorm_last_hip_error() -> int:
    return int(load_library().rmsnorm_last_hip_error())


# ------------------------------------------------------- torch conveniences

def dtype_code(t) -> int:
    import torch
    codes = {torch.float32: RMSN_F32, torch.float16: RMSN_F16, torch.bfloat16: RMSN_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _rows(t, N):
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.dim() < 1 or t.shape[-1] != N:
        raise ValueError(f"last dimension {tuple(t.shape)[-1:]} != N = {N}")
    return t.numel() // N


def _args(like, *specs):
    """Check the tensors a convenience hands to the library before any call:
    each spec is (tensor or None, name, numel or None, dtype or None). Every
    tensor must be contiguous, hold the stated number of elements and dtype,
    and sit on ``like``'s device (a GPU)."""
    for t, name, numel, dtype in specs:
        if t is None:
            continue
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    for t, name, _, _ in specs:
        if t is not None and (t.device != like.device or not t.is_cuda):
            raise ValueError(f"{name}: on {t.device}; every tensor must be on the same GPU "
                             f"(x is on {like.device})")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(status, where):
    if status != RMSN_OK:
        raise RMSNormError(status, where)


def fwd(x, gamma, eps: float = 1e-5, *, want_rstd: bool = False, out=None, rstd=None,
        stream=None):
    """y = RMSNorm(x) over the last dimension; returns (y, rstd or None)."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    _args(x, (x, "x", None, None), (gamma, "gamma", N, None), (out, "out", M * N, x.dtype),
          (rstd, "rstd", M, torch.float32))
    y = torch.empty_like(x) if out is None else out
    if want_rstd and rstd is None:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(rmsnorm_fwd(x, gamma, y, rstd, M, N, eps, dtype_code(x), dtype_code(gamma), stream),
           "rmsnorm_fwd")
    return y, rstd


def fused_add_fwd(x, residual, gamma, eps: float = 1e-5, *, want_rstd: bool = False, out=None,
                  rstd=None, stream=None):
    """residual <- x + residual (rounded), y = RMSNorm(residual); returns (y, rstd)."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    if residual.shape != x.shape or residual.dtype != x.dtype:
        raise ValueError("residual must match x in shape and dtype")
    _args(x, (x, "x", None, None), (residual, "residual", M * N, x.dtype),
          (gamma, "gamma", N, None), (out, "out", M * N, x.dtype), (rstd, "rstd", M, torch.float32))
    y = torch.empty_like(x) if out is None else out
    if want_rstd and rstd is None:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(rmsnorm_fused_add_fwd(x, residual, gamma, y, rstd, M, N, eps, dtype_code(x),
                                 dtype_code(gamma), stream), "rmsnorm_fused_add_fwd")
    return y, rstd


def quant_fwd(x, gamma, eps: float = 1e-5, *, scale=None, residual=None, want_rstd: bool = False,
              out=None, rstd=None, stream=None):
    """fp8 e4m3 output. With ``scale`` (a 1-element fp32 device tensor) every
    row uses it; without, per-row scales are computed and returned. With
    ``residual`` the fused add runs first (residual <- x + residual).
    Returns (q as torch.uint8 codes, scale, rstd or None)."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    if residual is not None and (residual.shape != x.shape or residual.dtype != x.dtype):
        raise ValueError("residual must match x in shape and dtype")
    _args(x, (x, "x", None, None), (residual, "residual", M * N, x.dtype),
          (gamma, "gamma", N, None), (out, "out", M * N, torch.uint8),
          (scale, "scale", 1, torch.float32), (rstd, "rstd", M, torch.float32))
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    mode = RMSN_QUANT_FP8_TENSOR if scale is not None else RMSN_QUANT_FP8_ROW
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if want_rstd and rstd is None:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(rmsnorm_quant_fwd(x, residual, gamma, q, scale, mode, rstd, M, N, eps, dtype_code(x),
                             dtype_code(gamma), stream), "rmsnorm_quant_fwd")
    return q, scale, rstd


def qk_fwd(q, k, q_gamma, k_gamma=None, eps: float = 1e-6, *, stream=None):
    """Per-head RMSNorm of q [T, Hq, D] and k [T, Hk, D] (k may be None), in
    place. Head vectors must be contiguous and heads D apart (views of a
    fused QKV buffer qualify); tokens may be strided. Returns (q, k)."""
    import torch

    def layout(t, name):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name}: expected [T, H, D] with contiguous heads")
        return t.shape[0], t.shape[1], t.shape[2], t.stride(0)

    T, Hq, D, sq = layout(q, "q")
    Hk, sk = 0, 0
    if k is not None:
        Tk, Hk, Dk, sk = layout(k, "k")
        if (Tk, Dk) != (T, D) or k.dtype != q.dtype:
            raise ValueError("k must match q in tokens, head_dim and dtype")
        if k_gamma is None:
            raise ValueError("k_gamma is required with k")
    for t, name in ((q, "q"), (k, "k")):
        if t is not None and (t.device != q.device or not t.is_cuda):
            raise ValueError(f"{name}: on {t.device}; q and k must be on the same GPU")
    _args(q, (q_gamma, "q_gamma", D, None),
          (k_gamma if k is not None else None, "k_gamma", D, q_gamma.dtype))
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    _check(rmsnorm_qk_fwd(q, k, q_gamma, k_gamma if k is not None else None, T, Hq, Hk, D, sq, sk,
                          eps, dtype_code(q), dtype_code(q_gamma), stream), "rmsnorm_qk_fwd")
    return q, k


def layernorm(x, gamma, beta=None, eps: float = 1e-5, *, want_stats: bool = False, out=None,
              stream=None):
    """LayerNorm over the last dimension; returns (y, mean, rstd), the
    statistics fp32 [rows] when want_stats, else None."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    _args(x, (x, "x", None, None), (gamma, "gamma", N, None), (beta, "beta", N, gamma.dtype),
          (out, "out", M * N, x.dtype))
    y = torch.empty_like(x) if out is None else out
    mean = rstd = None
    if want_stats:
        mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(layernorm_fwd(x, gamma, beta, y, mean, rstd, M, N, eps, dtype_code(x),
                         dtype_code(gamma), stream), "layernorm_fwd")
    return y, mean, rstd


def mx_quant_fwd(x, gamma, eps: float = 1e-5, *, fp4: bool = False, residual=None,
                 want_rstd: bool = False, stream=None):
    """MX block-scaled output (N % 32 == 0): returns (q uint8 codes, E8M0 scale
    codes [rows, N / 32] uint8, rstd or None); MXFP4 packs two codes per byte."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    if residual is not None and (residual.shape != x.shape or residual.dtype != x.dtype):
        raise ValueError("residual must match x in shape and dtype")
    _args(x, (x, "x", None, None), (residual, "residual", M * N, x.dtype),
          (gamma, "gamma", N, None))
    qshape = x.shape[:-1] + ((N // 2,) if fp4 else (N,))
    q = torch.empty(qshape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(x.shape[:-1] + (N // 32,), dtype=torch.uint8, device=x.device)
    rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if want_rstd else None
    mode = RMSN_QUANT_MXFP4 if fp4 else RMSN_QUANT_MXFP8
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(rmsnorm_quant_fwd(x, residual, gamma, q, scale, mode, rstd, M, N, eps, dtype_code(x),
                             dtype_code(gamma), stream), "rmsnorm_quant_fwd")
    return q, scale, rstd


def bwd(dy, x, rstd, gamma, *, dx=None, dgamma=None, workspace=None, stream=None):
    """Returns (dx, dgamma fp32). The workspace is allocated if not given."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    _args(x, (x, "x", None, None), (dy, "dy", M * N, x.dtype), (rstd, "rstd", M, torch.float32),
          (gamma, "gamma", N, None), (dx, "dx", M * N, x.dtype),
          (dgamma, "dgamma", N, torch.float32), (workspace, "workspace", None, None))
    dx = torch.empty_like(x) if dx is None else dx
    dgamma = torch.empty(N, dtype=torch.float32, device=x.device) if dgamma is None else dgamma
    ws_bytes = rmsnorm_bwd_workspace_size(M, N)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(rmsnorm_bwd(dy, x, rstd, gamma, dx, dgamma, workspace, _nbytes(workspace), M, N,
                       dtype_code(x), dtype_code(gamma), stream), "rmsnorm_bwd")
    return dx, dgamma


def fused_add_bwd(dy, h, rstd, gamma, dresidual=None, *, dh=None, dgamma=None, workspace=None,
                  stream=None):
    """Backward of fused_add_fwd: returns (dh, dgamma); dh is the gradient of
    both x and the residual. ``h`` is the residual buffer after the forward."""
    import torch
    N = gamma.numel()
    M = _rows(h, N)
    for t in (dy, dresidual):
        if t is not None and (t.shape != h.shape or t.dtype != h.dtype):
            raise ValueError("dy / dresidual must match h in shape and dtype")
    _args(h, (h, "h", None, None), (dy, "dy", M * N, h.dtype), (rstd, "rstd", M, torch.float32),
          (gamma, "gamma", N, None), (dresidual, "dresidual", M * N, h.dtype),
          (dh, "dh", M * N, h.dtype), (dgamma, "dgamma", N, torch.float32),
          (workspace, "workspace", None, None))
    dh = torch.empty_like(h) if dh is None else dh
    dgamma = torch.empty(N, dtype=torch.float32, device=h.device) if dgamma is None else dgamma
    ws_bytes = rmsnorm_bwd_workspace_size(M, N)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=h.device)
    stream = torch.cuda.current_stream(h.device) if stream is None else stream
    _check(rmsnorm_fused_add_bwd(dy, h, rstd, gamma, dresidual, dh, dgamma, workspace,
                                 _nbytes(workspace), M, N, dtype_code(h), dtype_code(gamma), stream),
           "rmsnorm_fused_add_bwd")
    return dh, dgamma


def layernorm_backward(dy, x, mean, rstd, gamma, *, want_dbeta: bool = True, dx=None,
                       workspace=None, stream=None):
    """LayerNorm backward with the forward's mean and rstd; returns
    (dx, dgamma fp32, dbeta fp32 or None)."""
    import torch
    N = gamma.numel()
    M = _rows(x, N)
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    _args(x, (x, "x", None, None), (dy, "dy", M * N, x.dtype), (mean, "mean", M, torch.float32),
          (rstd, "rstd", M, torch.float32), (gamma, "gamma", N, None),
          (dx, "dx", M * N, x.dtype), (workspace, "workspace", None, None))
    dx = torch.empty_like(x) if dx is None else dx
    dgamma = torch.empty(N, dtype=torch.float32, device=x.device)
    dbeta = torch.empty(N, dtype=torch.float32, device=x.device) if want_dbeta else None
    ws_bytes = layernorm_bwd_workspace_size(M, N)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    stream = torch.cuda.current_stream(x.device) if stream is None else stream
    _check(layernorm_bwd(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, workspace,
                         _nbytes(workspace), M, N, dtype_code(x), dtype_code(gamma), stream),
           "layernorm_bwd")
    return dx, dgamma, dbeta
