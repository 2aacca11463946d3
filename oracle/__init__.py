"""TEST INFRASTRUCTURE ONLY — the float64 CPU oracle of packed variable-length attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this package. It shares no code with the HIP path (``variable_length_flash_amd``) and imports
nothing from it; the two meet only in the seeded input generator, which holds none of the
method's arithmetic.

Everything here follows hanzo-kernel 0.2.42, ``src/packed.rs``:

* ``tile_table`` — the host-side ``layout`` function: for each sequence in order, one
  ``(sequence, first row)`` pair per ``br`` rows; zero-length sequences get none.
* ``visible_pairs`` — the number of (query, key) pairs one head computes: per row, the keys of
  its own sequence within the window (the masking of ``attend``'s online softmax).
* ``attend`` — the f64 composite ``attend_ref`` (mode "A") and the same with the matrix
  operands rounded as ``attend``'s query- and key-tile loads round them (mode "B"); the C
  source ``vlf_oracle.c`` states both definitions.
* ``attend_backward`` — the f64 gradient of ``sum(out * dout)`` with respect to qkv
  (``attend_back_ref``), in the same two modes; ``operands`` gives the score operands it is
  taken through.

Parity pins for every function live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libvlf_oracle.so")

F16, BF16 = 0, 1
DTYPES = {"fp16": F16, "f16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}
MODES = {"A": 0, "B": 1}

_lib = None


def _open(path):
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    lib.vlf_oracle_attend.argtypes = [
        p, p, p, ctypes.c_int64, p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_double, ctypes.c_int32, ctypes.c_int32, p, ctypes.c_int64,
        ctypes.c_int32, p, p,
    ]
    lib.vlf_oracle_attend.restype = ctypes.c_int
    lib.vlf_oracle_round.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p]
    lib.vlf_oracle_round.restype = ctypes.c_int
    lib.vlf_oracle_threads.argtypes = [ctypes.c_int32]
    lib.vlf_oracle_threads.restype = ctypes.c_int32
    lib.vlf_oracle_operands.argtypes = [
        p, p, p, ctypes.c_int64, p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_double, ctypes.c_int32, ctypes.c_int32, p, p,
    ]
    lib.vlf_oracle_operands.restype = ctypes.c_int
    return lib


def _load(path=None):
    """The oracle library (built on first use); ``path`` opens another build of the same source
    (the mutation tests use it)."""
    global _lib
    if path is not None:
        return _open(path)
    if _lib is None:
        if not os.path.exists(LIBRARY):
            from . import build as _build
            _build.build()
        _lib = _open(LIBRARY)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads(requested: int = 0) -> int:
    """Threads the oracle's parallel loops use (after setting ``requested`` if > 0)."""
    return int(_load().vlf_oracle_threads(int(requested)))


def round_to(x, dtype: str, *, library=None) -> np.ndarray:
    """Round float64 values to the storage type (round-to-nearest-even), as float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    rc = _load(library).vlf_oracle_round(_ptr(x), x.size, DTYPES[dtype], _ptr(y))
    if rc != 0:
        raise ValueError("bad dtype")
    return y


def attend(qkv, cos, sin, cu, heads: int, window: int, scale: float, *, mode: str = "B",
           dtype: str = "bf16", rows=None, nthreads: int = 0, library=None):
    """Oracle outputs for packed attention.

    qkv: [T, 3*heads*64] values of the storage type (any float array; widened to float32,
    which is exact for bf16/fp16). cos, sin: [P, 32]. cu: [S+1] int. window: 0 = every key of
    the sequence, W >= 1 = keys with |i - j| < W. rows: token indices to evaluate (None = all).

    Returns (out [n, heads*64] float64, lse [heads, n] float64) for the n requested tokens.
    """
    qkv = np.ascontiguousarray(qkv, dtype=np.float32)
    cos = np.ascontiguousarray(cos, dtype=np.float32)
    sin = np.ascontiguousarray(sin, dtype=np.float32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T = int(cu[-1])
    S = int(cu.shape[0] - 1)
    if qkv.shape != (T, 3 * heads * 64):
        raise ValueError(f"qkv shape {qkv.shape} != {(T, 3 * heads * 64)}")
    if cos.ndim != 2 or cos.shape[1] != 32 or sin.shape != cos.shape:
        raise ValueError("cos/sin must be [P, 32]")
    if rows is None:
        n = T
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = int(rows.shape[0])
        rows_p = _ptr(rows)
    out = np.zeros((n, heads * 64), dtype=np.float64)
    lse = np.zeros((n, heads), dtype=np.float64)
    rc = _load(library).vlf_oracle_attend(
        _ptr(qkv), _ptr(cos), _ptr(sin), cos.shape[0], _ptr(cu), S, T, heads, int(window),
        float(scale), MODES[mode], DTYPES[dtype], rows_p, n, int(nthreads), _ptr(out), _ptr(lse),
    )
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return out, np.ascontiguousarray(lse.T)


def operands(qkv, cos, sin, cu, heads: int, scale: float, *, mode: str = "B",
             dtype: str = "bf16", library=None):
    """The score operands (q~ [T, heads*64], k~ [T, heads*64], float64) of every token: the
    query rows rotated to their positions and scaled, the key rows rotated; in mode B rounded as
    ``attend``'s mode B rounds them. The scores are ``<q~_i, k~_j>``."""
    qkv = np.ascontiguousarray(qkv, dtype=np.float32)
    cos = np.ascontiguousarray(cos, dtype=np.float32)
    sin = np.ascontiguousarray(sin, dtype=np.float32)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    T, S = int(cu[-1]), int(cu.shape[0] - 1)
    if qkv.shape != (T, 3 * heads * 64):
        raise ValueError(f"qkv shape {qkv.shape} != {(T, 3 * heads * 64)}")
    q = np.zeros((T, heads * 64), dtype=np.float64)
    k = np.zeros((T, heads * 64), dtype=np.float64)
    rc = _load(library).vlf_oracle_operands(
        _ptr(qkv), _ptr(cos), _ptr(sin), cos.shape[0], _ptr(cu), S, T, heads, float(scale),
        MODES[mode], DTYPES[dtype], _ptr(q), _ptr(k))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return q, k


def attend_backward(qkv, cos, sin, cu, heads: int, window: int, scale: float, dout, *,
                    mode: str = "B", dtype: str = "bf16", library=None) -> np.ndarray:
    """Gradient of ``sum(out * dout)`` with respect to qkv, in float64 (hanzo-kernel 0.2.42
    src/packed.rs, ``attend_back_ref``, the f64 composite's gradient; ``attend_back`` computes
    the same quantities tile by tile).

    Per sequence and head, with the score operands q~ (rotated, scaled) and k~ (rotated) of
    ``operands``: s_ij = <q~_i, k~_j> over the visible keys, p = softmax_j(s), dp_ij =
    <dout_i, v_j>, ds_ij = p_ij (dp_ij - sum_j p_ij dp_ij). Then dv_j = sum_i p_ij dout_i, the
    operand gradients dq~_i = sum_j ds_ij k~_j and dk~_j = sum_i ds_ij q~_i, taken back through
    the rotation (its transpose, [c s; -s c] per dimension pair at the row's position) and, for
    the query, the scale. Mode B differs from mode A only in the rounded operands.

    dout: [T, heads*64]. Returns dqkv [T, 3*heads*64] float64. Dense per (sequence, head):
    meant for test-sized batches.
    """
    cos64 = np.asarray(cos, dtype=np.float64)
    sin64 = np.asarray(sin, dtype=np.float64)
    x = np.asarray(qkv, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    hd = heads * 64
    qt, kt = operands(qkv, cos, sin, cu, heads, scale, mode=mode, dtype=dtype, library=library)
    g = np.zeros((T, 3 * hd), dtype=np.float64)

    def back(y, c, s):
        # transpose of the half-split rotation at each row's position
        y1, y2 = y[:, :32], y[:, 32:]
        return np.concatenate([y1 * c + y2 * s, y2 * c - y1 * s], axis=1)

    for si in range(len(cu) - 1):
        a, b = int(cu[si]), int(cu[si + 1])
        L = b - a
        if L == 0:
            continue
        c, s = cos64[:L], sin64[:L]
        visible = visible_mask(L, window)
        for h in range(heads):
            cols = slice(h * 64, (h + 1) * 64)
            q, k = qt[a:b, cols], kt[a:b, cols]
            v = x[a:b, 2 * hd + h * 64:2 * hd + (h + 1) * 64]
            o = do[a:b, cols]
            sc = np.where(visible, q @ k.T, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            p = e / e.sum(axis=1, keepdims=True)
            dp = o @ v.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq = ds @ k
            dk = ds.T @ q
            dv = p.T @ o
            g[a:b, h * 64:(h + 1) * 64] = back(dq, c, s) * scale
            g[a:b, hd + h * 64:hd + (h + 1) * 64] = back(dk, c, s)
            g[a:b, 2 * hd + h * 64:2 * hd + (h + 1) * 64] = dv
    return g


def tile_table(cu, br: int) -> np.ndarray:
    """``layout``'s tile table: [NT, 2] uint32 rows (sequence, first row), sequence-major."""
    cu = [int(x) for x in cu]
    tiles = []
    for s in range(len(cu) - 1):
        for i0 in range(0, cu[s + 1] - cu[s], br):
            tiles.append((s, i0))
    return np.array(tiles, dtype=np.uint32).reshape(-1, 2)


CAUSAL = 0x40000000  # ORed into a window value: the causal sliding window


def visible_mask(L: int, window: int) -> np.ndarray:
    """[L, L] bool: key j visible to row i of one sequence. window: 0 = every key, W >= 1 =
    |i - j| < W (hanzo-kernel 0.2.42 src/packed.rs, `attend`'s window); with CAUSAL set, j <= i
    and, for W >= 1, i - j < W (the array library page's sliding-window mask)."""
    w = int(window) & ~CAUSAL
    pos = np.arange(L)
    diff = pos[:, None] - pos[None, :]  # i - j
    visible = np.ones((L, L), dtype=bool) if w <= 0 else np.abs(diff) < w
    if int(window) & CAUSAL:
        visible &= diff >= 0
    return visible


def visible_pairs(cu, window: int) -> int:
    """(query, key) pairs one head computes: per row i of each sequence, the keys j of the same
    sequence the window admits, counted row by row."""
    w, causal = int(window) & ~CAUSAL, bool(int(window) & CAUSAL)
    total = 0
    cu = [int(x) for x in cu]
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L == 0:
            continue
        i = np.arange(L, dtype=np.int64)
        lo = np.maximum(0, i - w + 1) if w > 0 else np.zeros(L, dtype=np.int64)
        if causal:
            hi = i + 1
        else:
            hi = np.minimum(L, i + w) if w > 0 else np.full(L, L, dtype=np.int64)  # exclusive
        total += int((hi - lo).sum())
    return int(total)
