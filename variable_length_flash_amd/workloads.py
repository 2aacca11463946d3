"""Seeded synthetic inputs for packed variable-length attention.

This module only draws inputs. It does none of the attention's arithmetic, so both the HIP path's
callers and the float64 oracle can take their inputs from it.

* Sequence lengths are inclusive integer uniforms drawn first.
* ``qkv ~ N(0, 1)`` is drawn as float32 and rounded to the storage type with
  round-to-nearest-even.
* Rotary tables follow the recipe of the subject page's test helper ``tables``
  (hanzo-kernel 0.2.42, ``src/packed.rs``, test module): angle ``p / base^(2m/64)`` in float64,
  cosine and sine taken in float64, narrowed to float32 and then rounded to the storage type.
  Both the kernel and the oracle read the same rounded tables.

All draws use NumPy's ``Generator(PCG64(seed))``.

The five named workloads are the packed batches this library is measured and checked on: a tiny
two-sequence fp16 case, an encoder batch, a long sliding-window batch, many short sequences and
sixteen 8192-token sequences.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 64


@dataclass
class Workload:
    name: str
    lens: list
    heads: int
    dtype: str            # "bf16" | "fp16"
    window: int           # 0 = every key; W >= 1 = |i - j| < W
    base: float           # rotary base
    table_rows: int       # P, rows of the cos/sin tables
    scale: float = 0.125  # 64 ** -0.5
    seed: int = 0
    note: str = ""
    cu: np.ndarray = field(init=False)

    def __post_init__(self):
        self.cu = np.concatenate([[0], np.cumsum(np.asarray(self.lens, dtype=np.int64))]).astype(np.int32)

    @property
    def tokens(self) -> int:
        return int(self.cu[-1])

    @property
    def sequences(self) -> int:
        return len(self.lens)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float16


def _draw_lens(rng, count, lo, hi):
    return [int(x) for x in rng.integers(lo, hi + 1, size=count)]


def _draw_lens_to_total(rng, lo, hi, total):
    """Uniform lengths drawn until their sum reaches ``total``; the last one is cut so the
    lengths sum to ``total`` exactly."""
    lens = []
    while sum(lens) < total:
        lens.append(int(rng.integers(lo, hi + 1)))
    lens[-1] -= sum(lens) - total
    return lens


def tiny():
    return Workload("tiny", [100, 156], heads=2, dtype="fp16", window=0, base=1e4,
                    table_rows=256, seed=1, note="2 sequences (100, 156), T=256, H=2, fp16")


def encoder():
    rng = np.random.Generator(np.random.PCG64(2))
    lens = _draw_lens(rng, 64, 32, 512)
    return Workload("encoder", lens, heads=12, dtype="bf16", window=0, base=1e4,
                    table_rows=512, seed=2, note="64 sequences, lengths U{32..512}, H=12, bf16")


def sliding():
    rng = np.random.Generator(np.random.PCG64(3))
    lens = _draw_lens_to_total(rng, 512, 8192, 65536)
    return Workload("sliding", lens, heads=12, dtype="bf16", window=128, base=1.6e5,
                    table_rows=8192, seed=3,
                    note="lengths U{512..8192} packed to T=65536, H=12, bf16, W=128")


def many_short():
    rng = np.random.Generator(np.random.PCG64(4))
    lens = _draw_lens(rng, 1024, 1, 64)
    return Workload("many_short", lens, heads=16, dtype="fp16", window=0, base=1e4,
                    table_rows=64, seed=4, note="1024 sequences, lengths U{1..64}, H=16, fp16")


def long():
    return Workload("long", [8192] * 16, heads=16, dtype="bf16", window=0, base=1.6e5,
                    table_rows=8192, seed=5, note="16 sequences of 8192, T=131072, H=16, bf16")


WORKLOADS = {"tiny": tiny, "encoder": encoder, "sliding": sliding, "many_short": many_short,
             "long": long}


def custom(lens, heads, dtype="bf16", window=0, base=1e4, table_rows=None, seed=0, scale=0.125,
           name="custom"):
    table_rows = table_rows if table_rows is not None else max([1] + list(lens))
    return Workload(name, list(lens), heads=heads, dtype=dtype, window=window, base=base,
                    table_rows=table_rows, seed=seed, scale=scale)


def draw_qkv(w: Workload, seed=None) -> torch.Tensor:
    """qkv [T, 3*H*64] ~ N(0,1), drawn in float32 and rounded to the storage type (CPU tensor)."""
    rng = np.random.Generator(np.random.PCG64(w.seed * 1000 + 17 if seed is None else seed))
    x = rng.standard_normal((w.tokens, 3 * w.heads * HEAD_DIM), dtype=np.float32)
    return torch.from_numpy(x).to(w.torch_dtype)


def rope_tables(w: Workload):
    """cos, sin [P, 32] in the storage type (CPU tensors)."""
    p = np.arange(w.table_rows, dtype=np.float64)[:, None]
    m = np.arange(HEAD_DIM // 2, dtype=np.float64)[None, :]
    angle = p / np.power(w.base, 2.0 * m / HEAD_DIM)
    cos = torch.from_numpy(np.cos(angle).astype(np.float32)).to(w.torch_dtype)
    sin = torch.from_numpy(np.sin(angle).astype(np.float32)).to(w.torch_dtype)
    return cos, sin
