"""Brute-force dense attention for tiny packed batches (test helper, independent of the oracle).

One sequence at a time, the whole [L, L] score matrix is formed with an explicit boolean mask;
the softmax and the value product are matrix expressions. Rounding to the storage type uses the
library conversions (torch's bfloat16, NumPy's float16), not the oracle's own rounding code.
The rotation is the half-split one of hanzo-kernel 0.2.42 ``src/packed.rs`` (pairs m, m+32).
"""
import numpy as np
import torch


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    return x.astype(np.float16).astype(np.float64)


def rotate_block(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, mode: str, dtype: str,
                 scale: float) -> np.ndarray:
    """x [L, 64] rotated row by row with cos/sin [L, 32]."""
    if mode == "A":
        x = x.astype(np.float64)
        c = cos.astype(np.float64)
        s = sin.astype(np.float64)
        a, b = x[:, :32], x[:, 32:]
        return np.concatenate([a * c - b * s, a * s + b * c], axis=1) * 1.0
    x = x.astype(np.float32)
    c = cos.astype(np.float32)
    s = sin.astype(np.float32)
    a, b = x[:, :32], x[:, 32:]
    # the products of two storage-type values are exact in float32, so each difference or sum
    # below rounds once, like the kernel's float32 expression
    lo = (a * c - b * s) * np.float32(scale)
    hi = (a * s + b * c) * np.float32(scale)
    return to_storage(np.concatenate([lo, hi], axis=1), dtype)


def attend(qkv, cos, sin, lens, heads, window, scale, mode="A", dtype="bf16"):
    """Returns (out [T, heads*64], lse [heads, T]) in float64."""
    qkv = np.asarray(qkv, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    T = int(sum(lens))
    hd = heads * 64
    out = np.zeros((T, hd))
    lse = np.zeros((heads, T))
    start = 0
    for L in lens:
        if L == 0:
            continue
        mask = _mask(L, window)
        for h in range(heads):
            rows = qkv[start:start + L]
            q = rotate_block(rows[:, h * 64:(h + 1) * 64], cos[:L], sin[:L], mode, dtype,
                             scale if mode == "B" else 1.0)
            k = rotate_block(rows[:, hd + h * 64:hd + (h + 1) * 64], cos[:L], sin[:L], mode,
                             dtype, 1.0)
            v = rows[:, 2 * hd + h * 64:2 * hd + (h + 1) * 64]
            s = q @ k.T
            if mode == "A":
                s = s * scale
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            out[start:start + L, h * 64:(h + 1) * 64] = (e / z) @ v
            lse[h, start:start + L] = (m + np.log(z))[:, 0]
        start += L
    return out, lse


def scores(qkv, cos, sin, lens, heads, window, scale, mode="A", dtype="bf16"):
    """Per (sequence, head) masked score matrices [L, L] (-inf where invisible)."""
    qkv = np.asarray(qkv, dtype=np.float64)
    hd = heads * 64
    res = []
    start = 0
    for L in lens:
        pos = np.arange(L)
        mask = _mask(L, window)
        per_head = []
        for h in range(heads):
            rows = qkv[start:start + L]
            q = rotate_block(rows[:, h * 64:(h + 1) * 64], cos[:L], sin[:L], mode, dtype,
                             scale if mode == "B" else 1.0)
            k = rotate_block(rows[:, hd + h * 64:hd + (h + 1) * 64], cos[:L], sin[:L], mode,
                             dtype, 1.0)
            s = q @ k.T * (scale if mode == "A" else 1.0)
            per_head.append(np.where(mask, s, -np.inf))
        res.append(per_head)
        start += L
    return res


def tile_table(lens, br):
    """Tiles by direct enumeration of every row: a tile starts at each row whose position is a
    multiple of br."""
    out = []
    for s, L in enumerate(lens):
        for i in range(L):
            if i % br == 0:
                out.append((s, i))
    return np.array(out, dtype=np.uint32).reshape(-1, 2)


CAUSAL = 1 << 30  # the causal flag of a window value


def _visible(i, j, window):
    """Key j visible to row i: |i - j| < W (W = 0: always), and j <= i under the causal flag."""
    w = window & ~CAUSAL
    ok = w == 0 or abs(i - j) < w
    return ok and (j <= i if window & CAUSAL else True)


def _mask(L, window):
    return np.array([[_visible(i, j, window) for j in range(L)] for i in range(L)],
                    dtype=bool).reshape(L, L)


def pair_count(lens, window):
    """Visible (query, key) pairs per head by a double loop."""
    n = 0
    for L in lens:
        for i in range(L):
            for j in range(L):
                if _visible(i, j, window):
                    n += 1
    return n
