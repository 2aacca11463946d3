"""Per-shape schedule selection: the forward's tile height and path, and the backward's tile
height, measured once per shape on the caller's own inputs and cached.

hanzo-kernel 0.2.42 src/packed.rs, `attend_tuned` and `attend_back_tuned`: the page times every
usable tile on the first call for a (device, shape) key built from the head count, the window and
the token count and longest sequence rounded up to powers of two, and reuses the fastest for every
later call with that key. Here the candidates are the library's schedules (64-, 128- and
256-row tiles; for the forward also the direct path against the key-tile workspace), every one of
them a launch configuration the parity tests cover, and the key adds the device and the storage
type. Timing uses HIP events on the launch stream around library calls; no computation happens
here. The heuristic picks of ``binding.choose_br``, ``choose_prerotate`` and
``choose_backward_br`` (the library's schedule rule) remain the default when no tuning is asked
for.
"""
from __future__ import annotations

import json

import numpy as np

from . import binding

FORWARD_CANDIDATES = tuple((br, pre) for br in (64, 128, 256) for pre in (False, True))
BACKWARD_CANDIDATES = (64, 128, 256)

# (kind, key) -> {"pick": ..., "ms": {candidate name: ms}}
_cache: dict = {}


def pow2(n: int) -> int:
    """The smallest power of two >= n (1 for n <= 1)."""
    n = int(n)
    return 1 if n <= 1 else 1 << (n - 1).bit_length()


def shape_key(cu, heads: int, window: int, dtype: str, device: str = "") -> str:
    """The cache key of a batch: device, storage type, heads, window, and the token count and
    longest sequence rounded up to powers of two."""
    lens = np.diff(binding._host_cu(cu).astype(np.int64))
    tokens = int(lens.sum())
    longest = int(lens.max()) if lens.size else 0
    return (f"device={device},dtype={dtype},heads={int(heads)},window={int(window)},"
            f"tokens={pow2(tokens)},longest={pow2(longest)}")


def forward_name(br: int, prerotate: bool) -> str:
    return f"br{br}_{'workspace' if prerotate else 'direct'}"


def fastest(ms: dict) -> str:
    """The candidate with the smallest time (the first listed among equals)."""
    if not ms:
        raise ValueError("no candidate was timed")
    return min(ms, key=lambda k: (ms[k], list(ms).index(k)))


def cached(kind: str, key: str):
    return _cache.get((kind, key))


def clear() -> None:
    _cache.clear()


def save(path: str) -> None:
    """Write the cache as JSON (one entry per (kind, key))."""
    entries = [{"kind": k, "key": key, **v} for (k, key), v in sorted(_cache.items())]
    with open(path, "w") as f:
        json.dump(entries, f, indent=1)


def load(path: str) -> int:
    """Merge a cache written by ``save``; returns the number of entries read."""
    with open(path) as f:
        entries = json.load(f)
    for e in entries:
        pick = e["pick"]
        _cache[(e["kind"], e["key"])] = {"pick": tuple(pick) if isinstance(pick, list) else pick,
                                         "ms": dict(e["ms"])}
    return len(entries)


def _device_name(dev) -> str:
    import torch
    return torch.cuda.get_device_name(dev)


def _time(launch, iters: int, stream) -> float:
    """Milliseconds per launch: one untimed launch, then `iters` between two events."""
    import torch
    launch()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        launch()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / iters


def tune_forward(qkv, cos, sin, cu, heads: int, window: int = 0, scale: float = 0.125,
                 iters: int = 5):
    """(br, prerotate) of the fastest forward schedule for this batch's shape key, timing every
    candidate on the first call for the key."""
    import torch
    dev = qkv.device
    dtype = "bf16" if qkv.dtype == torch.bfloat16 else "fp16"
    key = shape_key(cu, heads, window, dtype, _device_name(dev))
    hit = cached("forward", key)
    if hit is not None:
        return tuple(hit["pick"])
    T = int(binding._host_cu(cu)[-1])
    out = torch.empty((T, heads * binding.HEAD_DIM), dtype=qkv.dtype, device=dev)
    lse = torch.empty((heads, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms = {}
    for br, pre in FORWARD_CANDIDATES:
        batch = binding.prepare(cu, dev, br, pre, window)
        ws = binding.new_workspace(batch, heads, dev) if pre else None
        ms[forward_name(br, pre)] = _time(
            lambda: binding.attend_into(batch, qkv, cos, sin, heads, window, scale, out, lse,
                                        workspace=ws), iters, stream)
    best = fastest(ms)
    pick = next(c for c in FORWARD_CANDIDATES if forward_name(*c) == best)
    _cache[("forward", key)] = {"pick": pick, "ms": ms}
    return pick


def tune_backward(qkv, cos, sin, cu, heads: int, out, lse, dout, window: int = 0,
                  scale: float = 0.125, iters: int = 3) -> int:
    """The fastest backward tile height for this batch's shape key."""
    import torch
    dev = qkv.device
    dtype = "bf16" if qkv.dtype == torch.bfloat16 else "fp16"
    key = shape_key(cu, heads, window, dtype, _device_name(dev))
    hit = cached("backward", key)
    if hit is not None:
        return int(hit["pick"])
    cu_host = binding._host_cu(cu)
    T, S = int(cu_host[-1]), int(cu_host.shape[0] - 1)
    dqkv = torch.empty_like(qkv)
    ws = torch.empty(max(binding.backward_workspace_bytes(T, S, heads, br)
                         for br in BACKWARD_CANDIDATES), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms = {}
    for br in BACKWARD_CANDIDATES:
        batch = binding.prepare(cu, dev, br, False, window)
        ms[f"br{br}"] = _time(
            lambda: binding.attend_backward_into(batch, qkv, cos, sin, heads, window, scale, out,
                                                 lse, dout, dqkv, workspace=ws), iters, stream)
    pick = int(fastest(ms)[2:])
    _cache[("backward", key)] = {"pick": pick, "ms": ms}
    return pick


def attend_tuned(qkv, cos, sin, cu, heads: int, window: int = 0, scale: float = 0.125):
    """``binding.attend`` at the tuned schedule: (out, lse)."""
    br, pre = tune_forward(qkv, cos, sin, cu, heads, window, scale)
    return binding.attend(qkv, cos, sin, cu, heads, window, scale, br=br, prerotate=pre)


def attend_backward_tuned(qkv, cos, sin, cu, heads: int, out, lse, dout, window: int = 0,
                          scale: float = 0.125):
    """``binding.attend_backward`` at the tuned tile height: dqkv."""
    br = tune_backward(qkv, cos, sin, cu, heads, out, lse, dout, window, scale)
    batch = binding.prepare(cu, qkv.device, br, False, window)
    return binding.attend_backward(qkv, cos, sin, batch, heads, out, lse, dout, window, scale)
