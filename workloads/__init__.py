"""Seeded synthetic layer workloads for the GPTQ per-layer path.

This module only draws random inputs: it holds none of the method's
arithmetic.  Both the HIP path (through its tests and the benchmark) and the
fp64 oracle are fed from here, so they always see the same bytes.

The pages ask for calibration activations "collected from real data" and for
trained weights (aicassindra.com, "tm_gptq_math", sections "Post-training
quantization and the per-layer objective" and "A worked two-weight example");
neither is available, so every tensor below is a seeded synthetic stand-in
with the shapes and distributions of the five named workloads.

Seeding: one ``numpy.random.SeedSequence(seed)`` per workload, spawned in a
fixed order: one child per weight matrix (in layer order), then per distinct
calibration input one child for its shared factors and one child per token
chunk.  Every chunk is therefore reproducible on its own, which lets a
consumer stream a 65536-token input without holding it whole.

Dtypes: values are drawn in float32/float64 and then cast once to the stated
storage dtype (``float16`` or ``float32``); both sides consume the cast
values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

__all__ = [
    "XSpec",
    "LayerSpec",
    "Workload",
    "WORKLOADS",
    "get",
    "make_weight",
    "x_chunk",
    "x_chunks",
    "x_full",
    "custom",
]


@dataclasses.dataclass(frozen=True)
class XSpec:
    """One calibration input ``X`` of shape ``[d_in, n_tokens]`` (row-major,
    each input channel's tokens contiguous).

    kind:
      ``lowrank``   ``Z + A @ B / sqrt(rank)``, Z, A, B ~ N(0,1); A is drawn
                    once ([d_in, rank]), Z and B per chunk.
      ``relu``      ``max(0, N(0,1))``.
      ``student_t`` Student-t with ``nu`` degrees of freedom.
    outliers: number of channels (rows) multiplied by ``outlier_scale``,
      chosen once with ``rng.choice`` before the cast.
    dead_frac: fraction of channels set to exactly zero (after the draw).
    """

    key: str
    d_in: int
    n_tokens: int
    dtype: str  # "float16" | "float32"
    kind: str
    rank: int = 0
    outliers: int = 0
    outlier_scale: float = 20.0
    dead_frac: float = 0.0
    nu: float = 4.0
    chunk: int = 2048


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    d_out: int
    d_in: int
    dtype: str  # "float16" | "float32"
    std: float
    x_key: str


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    layers: Tuple[LayerSpec, ...]
    xs: Tuple[XSpec, ...]
    bits: int
    group_size: int  # 0 = one grid per row
    block_size: int
    damp: float = 0.01
    seed: int = 0

    def x(self, key: str) -> XSpec:
        for s in self.xs:
            if s.key == key:
                return s
        raise KeyError(key)

    # children: [w_0 .. w_{L-1}] + per X spec: [factors, chunk_0 .. chunk_{C-1}]
    def _children(self) -> Tuple[List[np.random.SeedSequence], Dict[str, Tuple[np.random.SeedSequence, List[np.random.SeedSequence]]]]:
        root = np.random.SeedSequence(self.seed)
        w_children = root.spawn(len(self.layers))
        x_children = {}
        for s in self.xs:
            n_chunks = (s.n_tokens + s.chunk - 1) // s.chunk
            kids = root.spawn(1 + n_chunks)
            x_children[s.key] = (kids[0], kids[1:])
        return w_children, x_children


def _lowrank_1(name: str, d_out: int, d_in: int, n: int, wdtype: str, xdtype: str, rank: int,
               bits: int, group: int, block: int, std: float, outliers: int = 0, chunk: int = 2048,
               description: str = "", seed: int = 0) -> Workload:
    xs = XSpec("x", d_in, n, xdtype, "lowrank", rank=rank, outliers=outliers, chunk=chunk)
    return Workload(name, description, (LayerSpec("w", d_out, d_in, wdtype, std, "x"),), (xs,),
                    bits, group, block, seed=seed)


def _decoder_block(seed: int = 0) -> Workload:
    n = 65536
    xs = (
        XSpec("x_qkv", 4096, n, "float16", "student_t"),
        XSpec("x_o", 4096, n, "float16", "student_t"),
        XSpec("x_gu", 4096, n, "float16", "student_t"),
        XSpec("x_down", 11008, n, "float16", "student_t"),
    )
    layers = (
        LayerSpec("q", 4096, 4096, "float16", 0.02, "x_qkv"),
        LayerSpec("k", 4096, 4096, "float16", 0.02, "x_qkv"),
        LayerSpec("v", 4096, 4096, "float16", 0.02, "x_qkv"),
        LayerSpec("o", 4096, 4096, "float16", 0.02, "x_o"),
        LayerSpec("gate", 11008, 4096, "float16", 0.02, "x_gu"),
        LayerSpec("up", 11008, 4096, "float16", 0.02, "x_gu"),
        LayerSpec("down", 4096, 11008, "float16", 0.015, "x_down"),
    )
    return Workload("decoder_block", "full decoder block (q,k,v,o,gate,up,down), 65536 Student-t(4) tokens, 4-bit g128, B=128",
                    layers, xs, bits=4, group_size=128, block_size=128, seed=seed)


WORKLOADS: Dict[str, Workload] = {
    "tiny": _lowrank_1("tiny", 64, 128, 512, "float32", "float32", 4, 4, 0, 32, 0.02, chunk=512,
                       description="W 64x128 fp32, X 128x512 fp32 (rank-4 factor), 4-bit per-row, B=32"),
    "attn_proj": _lowrank_1("attn_proj", 4096, 4096, 2048, "float16", "float16", 64, 4, 0, 128, 0.02,
                            description="W 4096x4096 fp16, X 4096x2048 fp16 (rank-64 factor), 4-bit per-row, B=128"),
    "attn_proj_g128": _lowrank_1("attn_proj_g128", 4096, 4096, 131072, "float16", "float16", 64, 4, 128, 128, 0.02,
                                 outliers=8,
                                 description="same layer, X 4096x131072 fp16 streamed in 2048-token chunks, 8 outlier channels x20, 4-bit g128, B=128"),
    "mlp_down": Workload("mlp_down", "W 4096x11008 fp16 (std 0.015), X 11008x16384 fp16 ReLU-like with 1% dead channels, 3-bit per-row, B=128",
                         (LayerSpec("w", 4096, 11008, "float16", 0.015, "x"),),
                         (XSpec("x", 11008, 16384, "float16", "relu", dead_frac=0.01),),
                         bits=3, group_size=0, block_size=128),
    "decoder_block": _decoder_block(),
    "small_proj": _lowrank_1("small_proj", 4096, 128, 2048, "float16", "float16", 16, 4, 0, 128, 0.02, seed=7,
                             description="W 4096x128 fp16, X 128x2048 fp16 (rank-16 factor), 4-bit per-row: a layer "
                                         "small enough for the greedy (per-row order) variant"),
}

# ``attn_proj_g128`` uses the very same weight matrix as ``attn_proj``: both
# draw it from child 0 of SeedSequence(0).


def get(name: str) -> Workload:
    return WORKLOADS[name]


def custom(d_out: int, d_in: int, n_tokens: int, *, bits: int = 4, group_size: int = 0, block_size: int = 128,
           wdtype: str = "float32", xdtype: str = "float32", kind: str = "lowrank", rank: int = 4,
           dead_frac: float = 0.0, outliers: int = 0, std: float = 0.02, chunk: int = 0, seed: int = 0,
           damp: float = 0.01) -> Workload:
    """A small single-layer workload of arbitrary shape (ragged parity cases)."""
    chunk = chunk or max(1, n_tokens)
    xs = XSpec("x", d_in, n_tokens, xdtype, kind, rank=rank, dead_frac=dead_frac, outliers=outliers, chunk=chunk)
    return Workload(f"custom_{d_out}x{d_in}x{n_tokens}", "custom", (LayerSpec("w", d_out, d_in, wdtype, std, "x"),),
                    (xs,), bits, group_size, block_size, damp=damp, seed=seed)


def make_weight(wl: Workload, layer: int = 0) -> np.ndarray:
    """Weight ``[d_out, d_in]`` ~ N(0, std^2), cast to the layer dtype."""
    spec = wl.layers[layer]
    w_children, _ = wl._children()
    rng = np.random.default_rng(w_children[layer])
    w = rng.standard_normal((spec.d_out, spec.d_in), dtype=np.float32) * np.float32(spec.std)
    return w.astype(spec.dtype)


def _x_state(wl: Workload, key: str):
    spec = wl.x(key)
    _, x_children = wl._children()
    fac_ss, chunk_ss = x_children[key]
    frng = np.random.default_rng(fac_ss)
    A = None
    if spec.kind == "lowrank":
        A = frng.standard_normal((spec.d_in, spec.rank))
    out_rows = None
    if spec.outliers:
        out_rows = np.sort(frng.choice(spec.d_in, size=spec.outliers, replace=False))
    dead_rows = None
    n_dead = int(np.floor(spec.dead_frac * spec.d_in))
    if n_dead:
        dead_rows = np.sort(frng.choice(spec.d_in, size=n_dead, replace=False))
    return spec, chunk_ss, A, out_rows, dead_rows


def dead_channels(wl: Workload, key: str = "x") -> np.ndarray:
    """Indices of the channels the generator zeroes (empty if none)."""
    _, _, _, _, dead_rows = _x_state(wl, key)
    return np.zeros(0, np.int64) if dead_rows is None else dead_rows


def outlier_channels(wl: Workload, key: str = "x") -> np.ndarray:
    _, _, _, out_rows, _ = _x_state(wl, key)
    return np.zeros(0, np.int64) if out_rows is None else out_rows


def x_chunk(wl: Workload, key: str, c: int, _state=None) -> np.ndarray:
    """Token chunk ``c`` of input ``key``: ``[d_in, chunk]`` in the stored dtype."""
    spec, chunk_ss, A, out_rows, dead_rows = _state or _x_state(wl, key)
    t0 = c * spec.chunk
    n = min(spec.chunk, spec.n_tokens - t0)
    if n <= 0:
        raise IndexError(c)
    rng = np.random.default_rng(chunk_ss[c])
    if spec.kind == "lowrank":
        z = rng.standard_normal((spec.d_in, n))
        b = rng.standard_normal((spec.rank, n))
        x = z + (A @ b) / np.sqrt(spec.rank)
    elif spec.kind == "relu":
        x = np.maximum(rng.standard_normal((spec.d_in, n), dtype=np.float32), np.float32(0))
    elif spec.kind == "student_t":
        if spec.nu != 4.0:
            raise ValueError("only nu=4 is drawn")
        # t_4 = Z / sqrt(V/4) with V ~ chi^2_4 = 2 (E1 + E2), E ~ Exp(1)
        z = rng.standard_normal((spec.d_in, n), dtype=np.float32)
        e = rng.standard_exponential((spec.d_in, n), dtype=np.float32)
        e += rng.standard_exponential((spec.d_in, n), dtype=np.float32)
        x = z * np.sqrt(np.float32(2.0) / e)
    else:
        raise ValueError(spec.kind)
    if out_rows is not None:
        x[out_rows] *= spec.outlier_scale
    if dead_rows is not None:
        x[dead_rows] = 0
    return x.astype(spec.dtype)


def n_chunks(wl: Workload, key: str) -> int:
    s = wl.x(key)
    return (s.n_tokens + s.chunk - 1) // s.chunk


def x_chunks(wl: Workload, key: str = "x") -> Iterator[np.ndarray]:
    st = _x_state(wl, key)
    for c in range(n_chunks(wl, key)):
        yield x_chunk(wl, key, c, st)


def x_full(wl: Workload, key: str = "x", out: Optional[np.ndarray] = None, workers: int = 0) -> np.ndarray:
    """Whole input ``[d_in, n_tokens]`` assembled from its chunks (drawn in a
    thread pool: each chunk has its own seed, so the result does not depend
    on the number of workers)."""
    import concurrent.futures
    import os
    s = wl.x(key)
    if out is None:
        out = np.empty((s.d_in, s.n_tokens), dtype=s.dtype)
    st = _x_state(wl, key)

    def fill(c):
        t0 = c * s.chunk
        ch = x_chunk(wl, key, c, st)
        out[:, t0:t0 + ch.shape[1]] = ch

    nc = n_chunks(wl, key)
    workers = workers or min(16, len(os.sched_getaffinity(0)), nc)
    if workers <= 1:
        for c in range(nc):
            fill(c)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nc)))
    return out
