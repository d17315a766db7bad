"""ctypes binding of ``libgptq_mi355x.so`` (the C ABI in ``include/gptq.h``).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every computation happens in the library's kernels.
There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq_mi355x.so")

GPTQ_OK, GPTQ_EINVAL, GPTQ_EUNSUPPORTED, GPTQ_EHIP, GPTQ_EWORKSPACE, GPTQ_ESCRATCH = 0, 1, 2, 3, 4, 5
GPTQ_F16, GPTQ_F32 = 0, 1

EXPORTS = (
    "gptq_hessian_accumulate",
    "gptq_hessian_set",
    "gptq_hessian_accumulate_chunks",
    "gptq_prepare_hinv_workspace",
    "gptq_prepare_hinv",
    "gptq_prepare_hinv_fp32_workspace",
    "gptq_prepare_hinv_fp32",
    "gptq_prepare_hinv_noalloc",
    "gptq_prepare_hinv_noalloc_max_din",
    "gptq_quantize_layer_workspace",
    "gptq_quantize_layer_split_workspace",
    "gptq_quantize_layer",
    "gptq_quantize_layer_split",
    "gptq_status_string",
    "gptq_packed_words",
    "gptq_pack_codes",
    "gptq_dequantize",
    "gptq_output_error",
    "gptq_propagate",
    "gptq_obq_workspace",
    "gptq_obq_quantize",
    "gptq_kernel_count",
    "gptq_kernel_name",
    "gptq_timing_enable",
    "gptq_timing_read",
)


class GptqError(RuntimeError):
    def __init__(self, fn: str, rc: int, msg: str):
        super().__init__(f"{fn} -> {rc} ({msg})")
        self.rc = rc


_lib: Optional[ctypes.CDLL] = None

_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and declare every signature of ``include/gptq.h``."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m post_weight_quantization_04_amd.build`")
    # torch ships its own HIP runtime under the same soname.  Loading torch
    # first makes the library bind to that one runtime, the one that owns the
    # device memory and streams handed in; loaded the other way round, the
    # process holds two runtimes and every launch on torch's buffers fails.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    sig = {
        "gptq_hessian_accumulate": (_i32, [_vp, _i64, _vp, _i32, _i64, _i64, _vp]),
        "gptq_hessian_set": (_i32, [_vp, _i64, _vp, _i32, _i64, _i64, _vp]),
        "gptq_hessian_accumulate_chunks": (_i32, [_vp, _i64, _vp, _i64, _i32, _i64, _i64, _i32, _vp]),
        "gptq_prepare_hinv_workspace": (_sz, [_i64]),
        "gptq_prepare_hinv": (_i32, [_vp, _i64, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "gptq_prepare_hinv_fp32_workspace": (_sz, [_i64]),
        "gptq_prepare_hinv_fp32": (_i32, [_vp, _i64, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "gptq_prepare_hinv_noalloc": (_i32, [_vp, _i64, ctypes.c_double, _vp, _vp, _vp, _vp, _vp]),
        "gptq_prepare_hinv_noalloc_max_din": (_i64, []),
        "gptq_quantize_layer_workspace": (_sz, [_i64, _i64, _i64]),
        "gptq_quantize_layer_split_workspace": (_sz, [_i64, _i64, _i64]),
        "gptq_quantize_layer": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
        "gptq_quantize_layer_split": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _sz, _vp]),
        "gptq_status_string": (ctypes.c_char_p, [_i32]),
        "gptq_packed_words": (_i64, [_i64, _i32]),
        "gptq_pack_codes": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp]),
        "gptq_dequantize": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i64, _vp, _i32, _vp]),
        "gptq_output_error": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
        "gptq_propagate": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp, _i64, _i32, _vp]),
        "gptq_obq_workspace": (_sz, [_i64]),
        "gptq_obq_quantize": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _sz, _vp]),
        "gptq_kernel_count": (_i32, []),
        "gptq_kernel_name": (ctypes.c_char_p, [_i32]),
        "gptq_timing_enable": (_i32, [_i32]),
        "gptq_timing_read": (_i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(rc: int) -> str:
    return load().gptq_status_string(rc).decode()


def _check(fn: str, rc: int) -> None:
    if rc != GPTQ_OK:
        raise GptqError(fn, rc, status_string(rc))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return GPTQ_F16
    if t.dtype == torch.float32:
        return GPTQ_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------
# the three entry points
# ---------------------------------------------------------------------------
def _hessian_call(fn: str, H, X, stream) -> None:
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    d_in, n = X.shape
    if H.shape != (d_in, d_in):
        raise ValueError("H shape")
    if not X.is_cuda:
        raise ValueError("device tensor expected")
    rc = getattr(load(), fn)(_ptr(H), d_in, X.data_ptr(), _dtype_code(X), n, X.stride(0), _stream(stream))
    _check(fn, rc)


def hessian_accumulate(H, X, stream=None) -> None:
    """``H[lower] += 2 X X^T`` for ``X: [d_in, n]`` (a 2-D view with unit
    column stride; row stride = ``X.stride(0)``)."""
    _hessian_call("gptq_hessian_accumulate", H, X, stream)


def hessian_set(H, X, stream=None) -> None:
    """``H[lower] = 2 X X^T`` (the old values not read; the strictly upper
    triangle not written), for the first token chunk."""
    _hessian_call("gptq_hessian_set", H, X, stream)


def hessian_chunks(H, Xs, set_first: bool = False, stream=None) -> None:
    """``H[lower] (=|+=) sum_c 2 X_c X_c^T`` over a list of token chunks of
    one shape, dtype and row stride (2-D views with unit column stride);
    ``set_first`` writes H from the first chunk instead of adding."""
    Xs = list(Xs)
    if not Xs:
        raise ValueError("no chunks")
    X0 = Xs[0]
    for X in Xs:
        if X.dim() != 2 or X.stride(1) != 1 or not X.is_cuda:
            raise ValueError("chunks must be 2-D device views with unit column stride")
        if X.shape != X0.shape or X.stride(0) != X0.stride(0) or X.dtype != X0.dtype:
            raise ValueError("chunks differ in shape, row stride or dtype")
    d_in, n = X0.shape
    if H.shape != (d_in, d_in):
        raise ValueError("H shape")
    ptrs = (ctypes.c_void_p * len(Xs))(*[X.data_ptr() for X in Xs])
    rc = load().gptq_hessian_accumulate_chunks(_ptr(H), d_in, ctypes.cast(ptrs, ctypes.c_void_p), len(Xs),
                                               _dtype_code(X0), n, X0.stride(0), int(bool(set_first)),
                                               _stream(stream))
    _check("gptq_hessian_accumulate_chunks", rc)


def prepare_hinv_workspace(d_in: int, fp32: bool = False) -> int:
    lib = load()
    return int(lib.gptq_prepare_hinv_fp32_workspace(d_in) if fp32 else lib.gptq_prepare_hinv_workspace(d_in))


def prepare_hinv(H, damp_frac: float, U, dead=None, info=None, lambda_out=None, workspace=None,
                 stream=None, fp32: bool = False) -> None:
    """``gptq_prepare_hinv`` (float64 factorization) or, with ``fp32``,
    ``gptq_prepare_hinv_fp32``."""
    d_in = H.shape[0]
    name = "gptq_prepare_hinv_fp32" if fp32 else "gptq_prepare_hinv"
    rc = getattr(load(), name)(_ptr(H), d_in, float(damp_frac), _ptr(U), _ptr(dead), _ptr(info),
                               _ptr(lambda_out), _ptr(workspace),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream))
    _check(name, rc)


def prepare_hinv_noalloc(H, damp_frac: float, U, dead=None, info=None, lambda_out=None, stream=None) -> None:
    """``gptq_prepare_hinv`` on the library's fixed device scratch (no workspace, no allocation)."""
    d_in = H.shape[0]
    rc = load().gptq_prepare_hinv_noalloc(_ptr(H), d_in, float(damp_frac), _ptr(U), _ptr(dead), _ptr(info),
                                          _ptr(lambda_out), _stream(stream))
    _check("gptq_prepare_hinv_noalloc", rc)


def prepare_hinv_noalloc_max_din() -> int:
    return int(load().gptq_prepare_hinv_noalloc_max_din())


def quantize_layer_workspace(d_out: int, d_in: int, block_size: int, split: bool = False) -> int:
    name = "gptq_quantize_layer_split_workspace" if split else "gptq_quantize_layer_workspace"
    return int(getattr(load(), name)(d_out, d_in, block_size))


def quantize_layer(W, U, dead, bits: int, group_size: int, block_size: int, codes, scales, zeros,
                   err_row=None, minmax=None, workspace=None, stream=None, split: bool = False) -> None:
    """``gptq_quantize_layer``, or ``gptq_quantize_layer_split`` (the lazy
    trailing update on split-precision bf16 products) with ``split``."""
    d_out, d_in = W.shape
    name = "gptq_quantize_layer_split" if split else "gptq_quantize_layer"
    rc = getattr(load(), name)(_ptr(W), _dtype_code(W), d_out, d_in, _ptr(U), _ptr(dead), int(bits),
                               int(group_size), int(block_size), _ptr(codes), _ptr(scales), _ptr(zeros),
                               _ptr(err_row), _ptr(minmax), _ptr(workspace),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream))
    _check(name, rc)


# ---------------------------------------------------------------------------
# few-bit storage, dequantization, output error
# ---------------------------------------------------------------------------
def packed_words(d_in: int, bits: int) -> int:
    return int(load().gptq_packed_words(d_in, int(bits)))


def pack_codes(codes, bits: int, packed, stream=None) -> None:
    d_out, d_in = codes.shape
    rc = load().gptq_pack_codes(_ptr(codes), d_out, d_in, int(bits), _ptr(packed), _stream(stream))
    _check("gptq_pack_codes", rc)


def dequantize(packed, bits: int, d_in: int, scales, zeros, group_size: int, out, stream=None) -> None:
    d_out = packed.shape[0]
    rc = load().gptq_dequantize(_ptr(packed), int(bits), d_out, d_in, _ptr(scales), _ptr(zeros), int(group_size),
                                _ptr(out), _dtype_code(out), _stream(stream))
    _check("gptq_dequantize", rc)


def output_error(W, dead, packed, bits: int, scales, zeros, group_size: int, err_row, lam, out_row,
                 stream=None) -> None:
    d_out, d_in = W.shape
    rc = load().gptq_output_error(_ptr(W), _dtype_code(W), _ptr(dead), _ptr(packed), int(bits), _ptr(scales),
                                  _ptr(zeros), int(group_size), d_out, d_in, _ptr(err_row), _ptr(lam),
                                  _ptr(out_row), _stream(stream))
    _check("gptq_output_error", rc)


def propagate(W_hat, X, Y, activation: int = 0, stream=None) -> None:
    """``Y = act(W_hat X)``: ``W_hat [d_out, d_in]`` f16 contiguous, ``X
    [d_in, n]`` and ``Y [d_out, n]`` f16 2-D views with unit column stride
    (row strides ``X.stride(0)``, ``Y.stride(0)``); activation 0 none, 1 ReLU."""
    for t in (X, Y):
        if t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
            raise ValueError("X and Y must be 2-D device views with unit column stride")
    d_out, d_in = W_hat.shape
    n = X.shape[1]
    if X.shape[0] != d_in or Y.shape != (d_out, n):
        raise ValueError("shapes")
    rc = load().gptq_propagate(_ptr(W_hat), _dtype_code(W_hat), d_out, d_in, X.data_ptr(), _dtype_code(X), n,
                               X.stride(0), Y.data_ptr(), Y.stride(0), int(activation), _stream(stream))
    _check("gptq_propagate", rc)


def obq_workspace(d_in: int) -> int:
    return int(load().gptq_obq_workspace(int(d_in)))


def obq_quantize(W, U, dead, bits: int, codes, scales, zeros, order=None, loss=None, workspace=None,
                 stream=None) -> None:
    d_out, d_in = W.shape
    rc = load().gptq_obq_quantize(_ptr(W), _dtype_code(W), d_out, d_in, _ptr(U), _ptr(dead), int(bits),
                                  _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(order), _ptr(loss),
                                  _ptr(workspace),
                                  workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                  _stream(stream))
    _check("gptq_obq_quantize", rc)


# ---------------------------------------------------------------------------
# kernel timing
# ---------------------------------------------------------------------------
def kernel_names() -> Tuple[str, ...]:
    lib = load()
    return tuple(lib.gptq_kernel_name(i).decode() for i in range(lib.gptq_kernel_count()))


def timing_enable(name: Optional[str]) -> None:
    idx = -1 if name is None else kernel_names().index(name)
    _check("gptq_timing_enable", load().gptq_timing_enable(idx))


def timing_read() -> Tuple[float, int]:
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check("gptq_timing_read", load().gptq_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
