"""Per-layer driver over the three C-ABI entry points.

Allocates device buffers with torch (memory and streams only) and enqueues
the library calls; it performs no arithmetic of its own.
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, Optional

from . import _lib


@dataclasses.dataclass
class Factor:
    U: "torch.Tensor"        # [d_in, d_in] float32, upper
    dead: "torch.Tensor"     # [d_in] uint8
    info: "torch.Tensor"     # [1] int32 (0 = ok)
    lam: "torch.Tensor"      # [1] float64


@dataclasses.dataclass
class Quantized:
    codes: "torch.Tensor"    # [d_out, d_in] uint8
    scales: "torch.Tensor"   # [d_out, n_groups] float32
    zeros: "torch.Tensor"    # [d_out, n_groups] int32
    err_row: "torch.Tensor"  # [d_out] float32
    minmax: "torch.Tensor"   # [d_out, n_groups, 2] float32


class Workspace:
    """Grow-only device scratch buffer shared by the calls of one stream."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        import torch
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def hessian(X, chunk: Optional[int] = None, H=None, stream=None):
    """``H = 2 X X^T`` (lower triangle) from a device ``X [d_in, N]``,
    streamed in token chunks of ``chunk`` (whole X if None): the first chunk
    sets the lower triangle, the others accumulate into it.  A new H has a
    zero upper triangle; that of a given H is left as it is."""
    import torch
    d_in, n = X.shape
    if H is None:
        H = torch.zeros((d_in, d_in), dtype=torch.float32, device=X.device)
    step = chunk or max(n, 1)
    full = [X[:, t0:t0 + step] for t0 in range(0, n - step + 1, step)]
    if len(full) > 1:
        # whole chunks in one call (summed before each add into H), then
        # the ragged last chunk
        _lib.hessian_chunks(H, full, set_first=True, stream=stream)
        t0 = len(full) * step
        if t0 < n:
            _lib.hessian_accumulate(H, X[:, t0:], stream=stream)
        return H
    _lib.hessian_set(H, X[:, 0:min(step, n)], stream=stream)
    for t0 in range(step, n, step):
        _lib.hessian_accumulate(H, X[:, t0:t0 + step], stream=stream)
    return H


def hessian_chunks(chunks: Iterable, d_in: int, device="cuda", H=None, stream=None):
    import torch
    if H is None:
        H = torch.zeros((d_in, d_in), dtype=torch.float32, device=device)
    for xc in chunks:
        _lib.hessian_accumulate(H, xc, stream=stream)
    return H


def prepare(H, damp_frac: float = 0.01, ws: Optional[Workspace] = None, out: Optional[Factor] = None,
            stream=None, fp32: bool = False) -> Factor:
    import torch
    d_in = H.shape[0]
    dev = H.device
    if out is None:
        out = Factor(torch.empty((d_in, d_in), dtype=torch.float32, device=dev),
                     torch.empty((d_in,), dtype=torch.uint8, device=dev),
                     torch.empty((1,), dtype=torch.int32, device=dev),
                     torch.empty((1,), dtype=torch.float64, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(_lib.prepare_hinv_workspace(d_in, fp32=fp32))
    _lib.prepare_hinv(H, damp_frac, out.U, out.dead, out.info, out.lam, buf, stream=stream, fp32=fp32)
    return out


def quantize(W, factor: Factor, bits: int, group_size: int, block_size: int, ws: Optional[Workspace] = None,
             out: Optional[Quantized] = None, use_dead: bool = True, stream=None, split: bool = False) -> Quantized:
    import torch
    d_out, d_in = W.shape
    dev = W.device
    ng = 1 if group_size == 0 else d_in // group_size
    if out is None:
        out = Quantized(torch.empty((d_out, d_in), dtype=torch.uint8, device=dev),
                        torch.empty((d_out, ng), dtype=torch.float32, device=dev),
                        torch.empty((d_out, ng), dtype=torch.int32, device=dev),
                        torch.empty((d_out,), dtype=torch.float32, device=dev),
                        torch.empty((d_out, ng, 2), dtype=torch.float32, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(_lib.quantize_layer_workspace(d_out, d_in, block_size, split=split))
    _lib.quantize_layer(W, factor.U, factor.dead if use_dead else None, bits, group_size, block_size, out.codes,
                        out.scales, out.zeros, out.err_row, out.minmax, buf, stream=stream, split=split)
    return out


def pack(codes, bits: int, stream=None):
    """Few-bit storage of ``codes [d_out, d_in]`` (uint32 words, see
    ``gptq_pack_codes``)."""
    import torch
    d_out, d_in = codes.shape
    packed = torch.empty((d_out, max(_lib.packed_words(d_in, bits), 1)), dtype=torch.int32, device=codes.device)
    _lib.pack_codes(codes, bits, packed, stream=stream)
    return packed


def dequantize(packed, bits: int, d_in: int, scales, zeros, group_size: int, dtype=None, stream=None):
    """``What = s (q - z)`` from packed codes, as ``dtype`` (float16 or float32)."""
    import torch
    out = torch.empty((packed.shape[0], d_in), dtype=dtype or torch.float32, device=packed.device)
    _lib.dequantize(packed, bits, d_in, scales, zeros, group_size, out, stream=stream)
    return out


def propagate(W_hat, X, relu: bool = False, out=None, stream=None):
    """The next layer's input from a quantized layer: ``Y = act(W_hat X)``
    in f16 (``gptq_propagate``); ``W_hat`` is the f16 dequantized layer."""
    import torch
    if out is None:
        out = torch.empty((W_hat.shape[0], X.shape[1]), dtype=torch.float16, device=X.device)
    _lib.propagate(W_hat, X, out, 1 if relu else 0, stream=stream)
    return out


def output_error(W, factor: Factor, q: Quantized, packed, bits: int, group_size: int, stream=None):
    """Per-row ``||dw X||^2`` from the loss identity (``gptq_output_error``)."""
    import torch
    out = torch.empty((W.shape[0],), dtype=torch.float32, device=W.device)
    _lib.output_error(W, factor.dead, packed, bits, q.scales, q.zeros, group_size, q.err_row, factor.lam, out,
                      stream=stream)
    return out


@dataclasses.dataclass
class GreedyQuantized:
    codes: "torch.Tensor"    # [d_out, d_in] uint8
    scales: "torch.Tensor"   # [d_out] float32
    zeros: "torch.Tensor"    # [d_out] int32
    order: "torch.Tensor"    # [d_out, d_in] int32: the column quantized at each step
    loss: "torch.Tensor"     # [d_out] float64: dw H_damped dw^T


def quantize_greedy(W, factor: Factor, bits: int, ws: Optional[Workspace] = None, use_dead: bool = True,
                    stream=None) -> GreedyQuantized:
    """Greedy-order (OBQ) quantization of a small layer (``d_in <= 128``,
    ``gptq_obq_quantize``)."""
    import torch
    d_out, d_in = W.shape
    dev = W.device
    out = GreedyQuantized(torch.empty((d_out, d_in), dtype=torch.uint8, device=dev),
                          torch.empty((d_out,), dtype=torch.float32, device=dev),
                          torch.empty((d_out,), dtype=torch.int32, device=dev),
                          torch.empty((d_out, d_in), dtype=torch.int32, device=dev),
                          torch.empty((d_out,), dtype=torch.float64, device=dev))
    ws = ws or Workspace(dev)
    buf = ws.get(_lib.obq_workspace(d_in))
    _lib.obq_quantize(W, factor.U, factor.dead if use_dead else None, bits, out.codes, out.scales, out.zeros,
                      out.order, out.loss, buf, stream=stream)
    return out
