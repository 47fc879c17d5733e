"""MI355X-native dense GEMM on gfx950 matrix cores: C = A . B, and the
generalised C = alpha * op(A) * op(B) + beta * C with fp32 or bf16 C; and 2-D
convolution (forward and filter gradient) as im2col + that GEMM.

A thin ctypes binding over the C ABI of ``include/gemm.h`` and
``include/conv.h`` (library
``libdense_gemm.so`` next to this file).  The functions of the same names take
the same arguments as the C entry points -- sizes, device pointers as
integers, leading dimensions and a stream handle -- and only marshal them;
every step of the product runs in the HIP kernels.  ``gemm`` is a convenience
over torch tensors (torch provides device memory and streams, nothing else).

The library is loaded on first use.  When it is missing this raises; there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdense_gemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_HIP = -2
GEMM_ERR_NO_DEVICE = -3
GEMM_ERR_OUT_OF_MEMORY = -4
GEMM_ERR_INTERNAL = -5
GEMM_ERR_CAPTURING = -6
GEMM_ERR_SCRATCH_LIMIT = -7
GEMM_SCRATCH_BYTES = 64 << 20
GEMM_DTYPE_F32 = 0
GEMM_DTYPE_BF16 = 1
GEMM_OP_N = 0
GEMM_OP_T = 1

# Every symbol include/gemm.h declares, with its ctypes signature.
_i64, _p, _int, _f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_GEMM_ARGS = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_GEMM_EX_ARGS = [_int, _int, _int, _int, _i64, _i64, _i64, _f, _p, _i64, _p, _i64, _f, _p, _i64, _p]
SIGNATURES = {
    "gemm_f32": (_int, _GEMM_ARGS),
    "gemm_bf16": (_int, _GEMM_ARGS),
    "gemm_status_string": (ctypes.c_char_p, [_int]),
    "gemm_num_configs": (_int, [_int]),
    "gemm_select_config": (_int, [_int, _i64, _i64, _i64]),
    "gemm_select_config_ex": (_int, [_int, _int, _int, _i64, _i64, _i64]),
    "gemm_config_name": (ctypes.c_char_p, [_int, _int]),
    "gemm_split_k": (_int, [_int, _int, _i64, _i64, _i64]),
    "gemm_split_k_ex": (_int, [_int, _int, _int, _int, _i64, _i64, _i64]),
    "gemm_f32_with_config": (_int, [_int, _int] + _GEMM_ARGS),
    "gemm_bf16_with_config": (_int, [_int, _int] + _GEMM_ARGS),
    "gemm_ex": (_int, _GEMM_EX_ARGS),
    "gemm_ex_with_config": (_int, [_int, _int] + _GEMM_EX_ARGS),
    "gemm_ex_noalloc": (_int, _GEMM_EX_ARGS),
    "gemm_config_layouts": (_int, [_int, _int]),
    "gemm_release_buffers": (_int, [_p]),
    "gemm_operand_copy_bytes": (_i64, [_int, _int, _int, _i64, _i64, _i64, _p, _i64, _p, _i64]),
}



class Conv2dParams(ctypes.Structure):
    """conv2d_params of include/conv.h."""
    _fields_ = [(name, ctypes.c_int64) for name in (
        "batch", "in_channels", "height", "width", "out_channels", "kernel_h", "kernel_w",
        "pad_h", "pad_w", "stride_h", "stride_w", "dilation_h", "dilation_w")]


_pp = ctypes.POINTER(Conv2dParams)
_pi64 = ctypes.POINTER(ctypes.c_int64)
SIGNATURES.update({
    "conv2d_output_size": (_int, [_pp, _pi64, _pi64]),
    "conv2d_workspace_size": (_i64, [_int, _pp]),
    "conv2d_im2col": (_int, [_int, _pp, _i64, _p, _p, _i64, _p]),
    "conv2d_fwd": (_int, [_int, _int, _pp, _p, _p, _p, _p, _i64, _p]),
    "conv2d_bwd_weight": (_int, [_int, _pp, _p, _p, _p, _p, _i64, _p]),
    "conv2d_fwd_implicit": (_int, [_int, _int, _pp, _p, _p, _p, _p]),
    "conv2d_bwd_weight_implicit": (_int, [_int, _pp, _p, _p, _p, _p]),
    "conv2d_fwd_implicit_ex": (_int, [_int, _int, _pp, _int, _p, _p, _p, _p]),
    "conv2d_bwd_weight_implicit_ex": (_int, [_int, _pp, _int, _p, _p, _p, _p]),
})

CONV_ADDR_DEFAULT, CONV_ADDR_ANALYTIC, CONV_ADDR_TABLE, CONV_ADDR_PADDED, CONV_ADDR_WINDOW = \
    0, 1, 2, 3, 4


class ConvNdParams(ctypes.Structure):
    """convnd_params of include/conv.h."""
    _fields_ = [(name, ctypes.c_int64) for name in (
        "batch", "in_channels", "out_channels", "ndim")] + \
        [(name, ctypes.c_int64 * 4) for name in ("size", "kernel", "pad", "stride", "dilation")]


_pnd = ctypes.POINTER(ConvNdParams)
SIGNATURES.update({
    "convnd_output_size": (_int, [_pnd, _pi64]),
    "convnd_workspace_size": (_i64, [_int, _pnd]),
    "convnd_im2col": (_int, [_int, _pnd, _i64, _p, _p, _i64, _p]),
    "convnd_fwd": (_int, [_int, _int, _pnd, _p, _p, _p, _p, _i64, _p]),
    "convnd_bwd_weight": (_int, [_int, _pnd, _p, _p, _p, _p, _i64, _p]),
    "convnd_fwd_implicit": (_int, [_int, _int, _pnd, _p, _p, _p, _p]),
    "convnd_bwd_weight_implicit": (_int, [_int, _pnd, _p, _p, _p, _p]),
    "convnd_fwd_implicit_ex": (_int, [_int, _int, _pnd, _int, _p, _p, _p, _p]),
    "convnd_bwd_weight_implicit_ex": (_int, [_int, _pnd, _int, _p, _p, _p, _p]),
})

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("gemm failed: %s (status %d)" % (gemm_status_string(status), status))
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "HIP library %s is missing: build it with `python -m dense_gemm_03_amd.build` "
            "(there is no CPU fallback)" % path)
    # One HIP runtime per process: torch ships its own libamdhip64 (same
    # soname), and device pointers and streams from torch are only valid in
    # that runtime.  Importing torch first makes the library bind to it instead
    # of loading a second runtime next to it.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - C callers without torch
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ---------------------------------------------------------------- C names --

def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load_library().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load_library().gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_with_config(cfg, split_k, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load_library().gemm_f32_with_config(cfg, split_k, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_with_config(cfg, split_k, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load_library().gemm_bf16_with_config(cfg, split_k, M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_ex(dtype_ab, dtype_c, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
            stream=None) -> int:
    return load_library().gemm_ex(dtype_ab, dtype_c, transa, transb, M, N, K, alpha, A, lda, B, ldb,
                                  beta, C, ldc, stream)


def gemm_ex_noalloc(dtype_ab, dtype_c, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                    ldc, stream=None) -> int:
    return load_library().gemm_ex_noalloc(dtype_ab, dtype_c, transa, transb, M, N, K, alpha, A, lda,
                                          B, ldb, beta, C, ldc, stream)


def gemm_ex_with_config(cfg, split_k, dtype_ab, dtype_c, transa, transb, M, N, K, alpha, A, lda, B,
                        ldb, beta, C, ldc, stream=None) -> int:
    return load_library().gemm_ex_with_config(cfg, split_k, dtype_ab, dtype_c, transa, transb, M, N,
                                              K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_release_buffers(stream=None) -> int:
    return load_library().gemm_release_buffers(stream)


def gemm_config_layouts(dtype: int, cfg: int) -> int:
    return load_library().gemm_config_layouts(dtype, cfg)


def gemm_status_string(status: int) -> str:
    return load_library().gemm_status_string(status).decode()


def gemm_num_configs(dtype: int) -> int:
    return load_library().gemm_num_configs(dtype)


def gemm_select_config(dtype: int, M: int, N: int, K: int) -> int:
    return load_library().gemm_select_config(dtype, M, N, K)


def gemm_select_config_ex(dtype: int, transa: int, transb: int, M: int, N: int, K: int) -> int:
    return load_library().gemm_select_config_ex(dtype, transa, transb, M, N, K)


def gemm_config_name(dtype: int, cfg: int):
    name = load_library().gemm_config_name(dtype, cfg)
    return name.decode() if name is not None else None


def gemm_split_k(dtype: int, cfg: int, M: int, N: int, K: int) -> int:
    return load_library().gemm_split_k(dtype, cfg, M, N, K)


def gemm_split_k_ex(dtype: int, cfg: int, transa: int, transb: int, M: int, N: int, K: int) -> int:
    return load_library().gemm_split_k_ex(dtype, cfg, transa, transb, M, N, K)


def gemm_operand_copy_bytes(dtype_ab, transa, transb, M, N, K, A, lda, B, ldb) -> int:
    return load_library().gemm_operand_copy_bytes(dtype_ab, transa, transb, M, N, K, A, lda, B,
                                                  ldb)


# ----------------------------------------------------------- torch helper --

def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor, got shape %s" % (tuple(t.shape),))
    rows, cols = t.shape
    if t.numel() == 0:
        return max(int(cols), 1)   # nothing is read or written: any stride will do
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (unit column stride)")
    return int(t.stride(0)) if rows > 1 else max(int(cols), 1)


def gemm(A, B, out=None, cfg: int | None = None, split_k: int = 0, stream=None, *,
         alpha: float = 1.0, beta: float = 0.0, transa: bool = False, transb: bool = False,
         out_dtype=None):
    """C = alpha * op(A) . op(B) + beta * C for CUDA (HIP) tensors.

    A and B are both float32 or both bfloat16, stored row-major with unit
    column stride (row strides become the leading dimensions): A is M x K, or
    K x M with ``transa``; B is K x N, or N x K with ``transb``.  C (``out``)
    is float32 or bfloat16 (``out_dtype``, default float32), M x N; it is
    created when not given (then ``beta`` must be 0).  With the defaults this
    is the plain product C = A . B (the gemm_f32 / gemm_bf16 entry points);
    otherwise gemm_ex runs.  Runs on ``stream`` (default: torch's current
    stream) and returns without synchronising."""
    import torch

    if A.dtype != B.dtype or A.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("A and B must both be float32 or both bfloat16")
    if A.device.type != "cuda" or B.device.type != "cuda":
        raise ValueError("A and B must be GPU tensors")
    if B.device != A.device:
        raise ValueError("A and B must be on the same GPU")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = (A.shape[1], A.shape[0]) if transa else (A.shape[0], A.shape[1])
    K2, N = (B.shape[1], B.shape[0]) if transb else (B.shape[0], B.shape[1])
    if K != K2:
        raise ValueError("inner dimensions differ: op(A) is %dx%d, op(B) is %dx%d" % (M, K, K2, N))
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("C must be float32 or bfloat16")
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing C (out=...)")
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if out.dtype != out_dtype or tuple(out.shape) != (M, N) or out.device != A.device:
        raise ValueError("out must be a %s (%d, %d) tensor on A's device" % (out_dtype, M, N))
    lda, ldb, ldc = _ld(A), _ld(B), _ld(out)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    bf16 = A.dtype == torch.bfloat16
    plain = (alpha == 1.0 and beta == 0.0 and not transa and not transb
             and out_dtype == torch.float32)
    # the library launches on the calling thread's current device
    with torch.cuda.device(A.device):
        if plain:
            args = (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, stream)
            if cfg is None:
                rc = (gemm_bf16 if bf16 else gemm_f32)(*args)
            else:
                rc = (gemm_bf16_with_config if bf16 else gemm_f32_with_config)(cfg, split_k,
                                                                                *args)
        else:
            args = (GEMM_DTYPE_BF16 if bf16 else GEMM_DTYPE_F32,
                    GEMM_DTYPE_BF16 if out_dtype == torch.bfloat16 else GEMM_DTYPE_F32,
                    GEMM_OP_T if transa else GEMM_OP_N, GEMM_OP_T if transb else GEMM_OP_N,
                    M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb, float(beta),
                    out.data_ptr(), ldc, stream)
            rc = gemm_ex(*args) if cfg is None else gemm_ex_with_config(cfg, split_k, *args)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return out


# ------------------------------------------------------------ convolution --

def conv2d_params(batch, in_channels, height, width, out_channels, kernel_h, kernel_w,
                  pad=(0, 0), stride=(1, 1), dilation=(1, 1)) -> Conv2dParams:
    return Conv2dParams(batch, in_channels, height, width, out_channels, kernel_h, kernel_w,
                        pad[0], pad[1], stride[0], stride[1], dilation[0], dilation[1])


def conv2d_output_size(params: Conv2dParams):
    """(status, P, Q)."""
    ph, pw = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = load_library().conv2d_output_size(ctypes.byref(params), ctypes.byref(ph), ctypes.byref(pw))
    return rc, ph.value, pw.value


def conv2d_workspace_size(dtype: int, params: Conv2dParams) -> int:
    return load_library().conv2d_workspace_size(dtype, ctypes.byref(params))


def conv2d_im2col(dtype, params, image, x, cols, ld_cols, stream=None) -> int:
    return load_library().conv2d_im2col(dtype, ctypes.byref(params), image, x, cols, ld_cols, stream)


def conv2d_fwd(dtype, dtype_y, params, x, w, y, workspace, workspace_bytes, stream=None) -> int:
    return load_library().conv2d_fwd(dtype, dtype_y, ctypes.byref(params), x, w, y, workspace,
                                     workspace_bytes, stream)


def conv2d_bwd_weight(dtype, params, x, dy, dw, workspace, workspace_bytes, stream=None) -> int:
    return load_library().conv2d_bwd_weight(dtype, ctypes.byref(params), x, dy, dw, workspace,
                                            workspace_bytes, stream)


def conv2d_fwd_implicit(dtype, dtype_y, params, x, w, y, stream=None) -> int:
    return load_library().conv2d_fwd_implicit(dtype, dtype_y, ctypes.byref(params), x, w, y, stream)


def conv2d_bwd_weight_implicit(dtype, params, x, dy, dw, stream=None) -> int:
    return load_library().conv2d_bwd_weight_implicit(dtype, ctypes.byref(params), x, dy, dw, stream)


def conv2d_fwd_implicit_ex(dtype, dtype_y, params, addressing, x, w, y, stream=None) -> int:
    return load_library().conv2d_fwd_implicit_ex(dtype, dtype_y, ctypes.byref(params), addressing,
                                                 x, w, y, stream)


def conv2d_bwd_weight_implicit_ex(dtype, params, addressing, x, dy, dw, stream=None) -> int:
    return load_library().conv2d_bwd_weight_implicit_ex(dtype, ctypes.byref(params), addressing,
                                                        x, dy, dw, stream)


def convnd_params(batch, in_channels, out_channels, size, kernel, pad=None, stride=None,
                  dilation=None) -> ConvNdParams:
    """ConvNdParams for len(size) spatial dimensions (unused entries 0)."""
    nd = len(size)
    pad = (0,) * nd if pad is None else tuple(pad)
    stride = (1,) * nd if stride is None else tuple(stride)
    dilation = (1,) * nd if dilation is None else tuple(dilation)
    if not 1 <= nd <= 4 or not all(len(v) == nd for v in (kernel, pad, stride, dilation)):
        raise ValueError("size, kernel, pad, stride and dilation need 1 to 4 entries each, alike")
    arr = lambda v: (ctypes.c_int64 * 4)(*(tuple(v) + (0,) * (4 - nd)))  # noqa: E731
    return ConvNdParams(batch, in_channels, out_channels, nd, arr(size), arr(kernel), arr(pad),
                        arr(stride), arr(dilation))


def convnd_output_size(params: ConvNdParams):
    """(status, (O_0, .., O_{ndim-1}))."""
    out = (ctypes.c_int64 * 4)()
    rc = load_library().convnd_output_size(ctypes.byref(params), out)
    return rc, tuple(out[i] for i in range(max(0, min(params.ndim, 4))))


def convnd_workspace_size(dtype: int, params: ConvNdParams) -> int:
    return load_library().convnd_workspace_size(dtype, ctypes.byref(params))


def convnd_im2col(dtype, params, image, x, cols, ld_cols, stream=None) -> int:
    return load_library().convnd_im2col(dtype, ctypes.byref(params), image, x, cols, ld_cols, stream)


def convnd_fwd(dtype, dtype_y, params, x, w, y, workspace, workspace_bytes, stream=None) -> int:
    return load_library().convnd_fwd(dtype, dtype_y, ctypes.byref(params), x, w, y, workspace,
                                     workspace_bytes, stream)


def convnd_bwd_weight(dtype, params, x, dy, dw, workspace, workspace_bytes, stream=None) -> int:
    return load_library().convnd_bwd_weight(dtype, ctypes.byref(params), x, dy, dw, workspace,
                                            workspace_bytes, stream)


def convnd_fwd_implicit(dtype, dtype_y, params, x, w, y, stream=None) -> int:
    return load_library().convnd_fwd_implicit(dtype, dtype_y, ctypes.byref(params), x, w, y, stream)


def convnd_bwd_weight_implicit(dtype, params, x, dy, dw, stream=None) -> int:
    return load_library().convnd_bwd_weight_implicit(dtype, ctypes.byref(params), x, dy, dw, stream)


def convnd_fwd_implicit_ex(dtype, dtype_y, params, addressing, x, w, y, stream=None) -> int:
    return load_library().convnd_fwd_implicit_ex(dtype, dtype_y, ctypes.byref(params), addressing,
                                                 x, w, y, stream)


def convnd_bwd_weight_implicit_ex(dtype, params, addressing, x, dy, dw, stream=None) -> int:
    return load_library().convnd_bwd_weight_implicit_ex(dtype, ctypes.byref(params), addressing,
                                                        x, dy, dw, stream)


def _pair(v):
    return (v, v) if isinstance(v, int) else tuple(v)


def _tuple_nd(v, nd):
    return (v,) * nd if isinstance(v, int) else tuple(v)


def _conv_setup(x, weight_shape, stride, padding, dilation):
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16) or x.device.type != "cuda" or x.dim() != 4:
        raise TypeError("x must be a 4-D float32 or bfloat16 GPU tensor (N, C, H, W)")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (channel-first)")
    co, ci, r, s = weight_shape
    if ci != x.shape[1]:
        raise ValueError("channel mismatch: x has %d, the filters %d" % (x.shape[1], ci))
    params = conv2d_params(x.shape[0], ci, x.shape[2], x.shape[3], co, r, s, _pair(padding),
                           _pair(stride), _pair(dilation))
    dtype = GEMM_DTYPE_BF16 if x.dtype == torch.bfloat16 else GEMM_DTYPE_F32
    rc, P, Q = conv2d_output_size(params)
    if rc != GEMM_OK:
        raise GemmError(rc)
    need = conv2d_workspace_size(dtype, params)
    return params, dtype, P, Q, need


def _workspace(workspace, need, device):
    import torch
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace of %d bytes needed" % need)
    return workspace


_ADDRESSING = {True: CONV_ADDR_DEFAULT, "analytic": CONV_ADDR_ANALYTIC, "table": CONV_ADDR_TABLE,
               "padded": CONV_ADDR_PADDED, "window": CONV_ADDR_WINDOW}


def conv2d(x, w, stride=1, padding=0, dilation=1, out_dtype=None, workspace=None, stream=None,
           implicit=False):
    """y = conv2d(x, w) (cross-correlation form, as torch.nn.functional.conv2d)
    through the im2col + GEMM path, or with ``implicit`` through the
    implicit-GEMM path (no convolution matrix): True (the library's address
    generation), "analytic", "table", "padded" or "window".  x (N, C_in, H, W) and w
    (C_out, C_in, R, S) are both float32 or both bfloat16; y is float32
    (default) or bfloat16.  The im2col workspace (one image's convolution
    matrix) is allocated when not given."""
    import torch
    if w.dtype != x.dtype or not w.is_contiguous() or w.dim() != 4:
        raise TypeError("w must be a contiguous 4-D tensor of x's dtype")
    if w.device != x.device:
        raise ValueError("x and w must be on the same GPU")
    params, dtype, P, Q, need = _conv_setup(x, tuple(w.shape), stride, padding, dilation)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    y = torch.empty((x.shape[0], w.shape[0], P, Q), dtype=out_dtype, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    dtype_y = GEMM_DTYPE_BF16 if out_dtype == torch.bfloat16 else GEMM_DTYPE_F32
    # the library launches on the calling thread's current device
    with torch.cuda.device(x.device):
        if implicit:
            rc = conv2d_fwd_implicit_ex(dtype, dtype_y, params, _ADDRESSING[implicit], x.data_ptr(),
                                        w.data_ptr(), y.data_ptr(), stream)
        else:
            ws = _workspace(workspace, need, x.device)
            rc = conv2d_fwd(dtype, dtype_y, params, x.data_ptr(), w.data_ptr(), y.data_ptr(),
                            ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return y


def conv2d_weight_grad(x, dy, weight_shape, stride=1, padding=0, dilation=1, workspace=None,
                       stream=None, implicit=False):
    """dw (float32, weight_shape) = the filter gradient of conv2d for input x
    and output gradient dy, through the im2col + GEMM path (or, with
    ``implicit`` -- True, "analytic", "table", "padded" or "window" -- the
    implicit-GEMM path)."""
    import torch
    params, dtype, P, Q, need = _conv_setup(x, tuple(weight_shape), stride, padding, dilation)
    if dy.dtype != x.dtype or not dy.is_contiguous() or \
            tuple(dy.shape) != (x.shape[0], weight_shape[0], P, Q):
        raise ValueError("dy must be a contiguous (N, C_out, P, Q) tensor of x's dtype")
    if dy.device != x.device:
        raise ValueError("x and dy must be on the same GPU")
    dw = torch.empty(tuple(weight_shape), dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    # the library launches on the calling thread's current device
    with torch.cuda.device(x.device):
        if implicit:
            rc = conv2d_bwd_weight_implicit_ex(dtype, params, _ADDRESSING[implicit], x.data_ptr(),
                                               dy.data_ptr(), dw.data_ptr(), stream)
        else:
            ws = _workspace(workspace, need, x.device)
            rc = conv2d_bwd_weight(dtype, params, x.data_ptr(), dy.data_ptr(), dw.data_ptr(),
                                   ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return dw


def _convnd_setup(x, weight_shape, stride, padding, dilation):
    import torch
    nd = x.dim() - 2
    if x.dtype not in (torch.float32, torch.bfloat16) or x.device.type != "cuda" or \
            not 1 <= nd <= 4:
        raise TypeError("x must be a float32 or bfloat16 GPU tensor (N, C, S_0 .. S_{D-1}), "
                        "D = 1 to 4")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (channel-first)")
    if len(weight_shape) != nd + 2 or weight_shape[1] != x.shape[1]:
        raise ValueError("filters must be (C_out, C_in, K_0 .. K_{D-1}) with x's C_in")
    params = convnd_params(x.shape[0], x.shape[1], weight_shape[0], tuple(x.shape[2:]),
                           tuple(weight_shape[2:]), _tuple_nd(padding, nd), _tuple_nd(stride, nd),
                           _tuple_nd(dilation, nd))
    dtype = GEMM_DTYPE_BF16 if x.dtype == torch.bfloat16 else GEMM_DTYPE_F32
    rc, out = convnd_output_size(params)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return params, dtype, out, convnd_workspace_size(dtype, params)


def conv_nd(x, w, stride=1, padding=0, dilation=1, out_dtype=None, workspace=None, stream=None,
            implicit=False):
    """y = convolution of x (N, C_in, S_0 .. S_{D-1}) with w (C_out, C_in,
    K_0 .. K_{D-1}), D = 1 to 4 (cross-correlation form, as torch's conv1d /
    conv2d / conv3d), through the im2col + GEMM path, or with ``implicit``
    (D <= 3) the implicit GEMM (True: the library's address generation,
    "analytic" or "padded").  x and w are both float32 or both bfloat16; y
    is float32 (default) or bfloat16."""
    import torch
    if w.dtype != x.dtype or not w.is_contiguous():
        raise TypeError("w must be a contiguous tensor of x's dtype")
    if w.device != x.device:
        raise ValueError("x and w must be on the same GPU")
    params, dtype, out, need = _convnd_setup(x, tuple(w.shape), stride, padding, dilation)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    y = torch.empty((x.shape[0], w.shape[0]) + out, dtype=out_dtype, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    dtype_y = GEMM_DTYPE_BF16 if out_dtype == torch.bfloat16 else GEMM_DTYPE_F32
    # the library launches on the calling thread's current device
    with torch.cuda.device(x.device):
        if implicit:
            rc = convnd_fwd_implicit_ex(dtype, dtype_y, params, _ADDRESSING[implicit], x.data_ptr(),
                                        w.data_ptr(), y.data_ptr(), stream)
        else:
            ws = _workspace(workspace, need, x.device)
            rc = convnd_fwd(dtype, dtype_y, params, x.data_ptr(), w.data_ptr(), y.data_ptr(),
                            ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return y


def conv_nd_weight_grad(x, dy, weight_shape, stride=1, padding=0, dilation=1, workspace=None,
                        stream=None, implicit=False):
    """dw (float32, weight_shape) = the filter gradient of conv_nd for input x
    and output gradient dy, through the im2col + GEMM path (or, with
    ``implicit`` -- True, "analytic" or "padded" -- and D <= 3, the implicit
    GEMM)."""
    import torch
    params, dtype, out, need = _convnd_setup(x, tuple(weight_shape), stride, padding, dilation)
    if dy.dtype != x.dtype or not dy.is_contiguous() or \
            tuple(dy.shape) != (x.shape[0], weight_shape[0]) + out:
        raise ValueError("dy must be a contiguous (N, C_out, O_0 ..) tensor of x's dtype")
    if dy.device != x.device:
        raise ValueError("x and dy must be on the same GPU")
    dw = torch.empty(tuple(weight_shape), dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    # the library launches on the calling thread's current device
    with torch.cuda.device(x.device):
        if implicit:
            rc = convnd_bwd_weight_implicit_ex(dtype, params, _ADDRESSING[implicit], x.data_ptr(),
                                               dy.data_ptr(), dw.data_ptr(), stream)
        else:
            ws = _workspace(workspace, need, x.device)
            rc = convnd_bwd_weight(dtype, params, x.data_ptr(), dy.data_ptr(), dw.data_ptr(),
                                   ws.data_ptr(), ws.numel() * ws.element_size(), stream)
    if rc != GEMM_OK:
        raise GemmError(rc)
    return dw
