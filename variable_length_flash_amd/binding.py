"""ctypes binding of libvlf.so (declared in include/vlf.h): argument marshalling only.

Every step of the forward runs in the library's gfx950 kernels. PyTorch supplies device memory
and the current HIP stream. When the library is missing this module raises; there is no other
implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libvlf.so")

VLF_OK, VLF_EINVAL, VLF_EUNSUPPORTED, VLF_EHIP = 0, -1, -2, -3
VLF_F16, VLF_BF16 = 0, 1
HEAD_DIM = 64

# every function include/vlf.h declares
EXPORTS = ("vlf_version", "vlf_last_error", "vlf_tile_count", "vlf_tile_table", "vlf_launch_table",
           "vlf_visible_pairs", "vlf_workspace_bytes", "vlf_schedule_rule", "vlf_typical_length",
           "vlf_choose_schedule", "vlf_choose_backward", "vlf_forward_kernel", "vlf_attend",
           "vlf_attend_static", "vlf_rotate_keys", "vlf_attend_rotated",
           "vlf_backward_workspace_bytes", "vlf_attend_backward", "vlf_rotate_qkv")


class VlfError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"vlf status {status}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return LIBRARY


def load_library():
    """Open libvlf.so (built by ``variable_length_flash_amd.build``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise VlfError(VLF_EHIP, f"{LIBRARY} is not built; run python -m "
                                 "variable_length_flash_amd.build")
    lib = ctypes.CDLL(LIBRARY)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.vlf_version.argtypes = []
    lib.vlf_version.restype = i32
    lib.vlf_last_error.argtypes = []
    lib.vlf_last_error.restype = ctypes.c_char_p
    lib.vlf_tile_count.argtypes = [p, i32, i32, i32, p, p]
    lib.vlf_tile_count.restype = ctypes.c_int
    lib.vlf_tile_table.argtypes = [p, i32, i32, i32, p, i64]
    lib.vlf_tile_table.restype = ctypes.c_int
    lib.vlf_launch_table.argtypes = [p, i32, i32, i32, i32, i32, p, i64]
    lib.vlf_launch_table.restype = ctypes.c_int
    lib.vlf_visible_pairs.argtypes = [p, i32, i32, i32, p]
    lib.vlf_visible_pairs.restype = ctypes.c_int
    lib.vlf_workspace_bytes.argtypes = [i32, i32, i32, p]
    lib.vlf_workspace_bytes.restype = ctypes.c_int
    lib.vlf_schedule_rule.argtypes = [i32, ctypes.c_double, i32, i32, p, p, p]
    lib.vlf_schedule_rule.restype = ctypes.c_int
    lib.vlf_typical_length.argtypes = [p, i32, i32, p]
    lib.vlf_typical_length.restype = ctypes.c_int
    lib.vlf_choose_schedule.argtypes = [p, i32, i32, i32, i32, p, p, p, p]
    lib.vlf_choose_schedule.restype = ctypes.c_int
    lib.vlf_choose_backward.argtypes = [p, i32, i32, i32, i32, p, p]
    lib.vlf_choose_backward.restype = ctypes.c_int
    lib.vlf_forward_kernel.argtypes = [i32, i32, i32, i32]
    lib.vlf_forward_kernel.restype = ctypes.c_char_p
    lib.vlf_attend.argtypes = [p, p, p, i32, i32, p, p, i32, i32, i32, i32, i32, i32,
                               ctypes.c_float, i32, p, i64, p, p, p]
    lib.vlf_attend.restype = ctypes.c_int
    lib.vlf_attend_rotated.argtypes = lib.vlf_attend.argtypes
    lib.vlf_attend_rotated.restype = ctypes.c_int
    lib.vlf_attend_static.argtypes = [p, p, p, i32, i32, p, p, i32, i32, i32, i32, i32, i32,
                                      ctypes.c_float, i32, p, p, p]
    lib.vlf_attend_static.restype = ctypes.c_int
    lib.vlf_rotate_keys.argtypes = [p, p, p, i32, i32, p, i32, i32, i32, i32, p, i64, p]
    lib.vlf_rotate_keys.restype = ctypes.c_int
    lib.vlf_backward_workspace_bytes.argtypes = [i32, i32, i32, i32, p]
    lib.vlf_backward_workspace_bytes.restype = ctypes.c_int
    lib.vlf_attend_backward.argtypes = [p, p, p, i32, i32, p, p, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_float, i32, p, p, p, p, i64, p, p]
    lib.vlf_attend_backward.restype = ctypes.c_int
    lib.vlf_rotate_qkv.argtypes = [p, p, p, i32, i32, p, p, i32, i32, i32, i32, i32,
                                   ctypes.c_float, i32, p, p]
    lib.vlf_rotate_qkv.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != VLF_OK:
        raise VlfError(status, load_library().vlf_last_error().decode())


def _host_cu(cu) -> np.ndarray:
    try:
        import torch
        if isinstance(cu, torch.Tensor):
            cu = cu.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    arr = np.asarray(cu)
    if arr.ndim != 1 or arr.shape[0] < 1:
        raise VlfError(VLF_EINVAL, "cu must be a 1-D sequence of S+1 offsets")
    if arr.size and (arr.min() < np.iinfo(np.int32).min or arr.max() > np.iinfo(np.int32).max):
        raise VlfError(VLF_EINVAL, "cu does not fit int32")
    return np.ascontiguousarray(arr, dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def tile_count(cu, br: int):
    """(num_tiles, max_len) for ``br``-row tiles of the packed batch ``cu``."""
    cu = _host_cu(cu)
    n, m = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().vlf_tile_count(_ptr(cu), cu.shape[0] - 1, int(cu[-1]), br,
                                         ctypes.byref(n), ctypes.byref(m)))
    return n.value, m.value


def tile_table(cu, br: int) -> np.ndarray:
    """The tile table [NT, 2] uint32 of (sequence, first row) pairs, from the library."""
    cu = _host_cu(cu)
    n, _ = tile_count(cu, br)
    table = np.zeros((n, 2), dtype=np.uint32)
    _check(load_library().vlf_tile_table(_ptr(cu), cu.shape[0] - 1, int(cu[-1]), br,
                                          _ptr(table), 2 * n))
    return table


def launch_table(cu, br: int, prerotate: bool = False, window: int = 0) -> np.ndarray:
    """The tile table in the library's launch order for this schedule (vlf_launch_table): the
    entries of ``tile_table`` permuted, [NT, 2] uint32."""
    cu = _host_cu(cu)
    n, _ = tile_count(cu, br)
    table = np.zeros((n, 2), dtype=np.uint32)
    _check(load_library().vlf_launch_table(_ptr(cu), cu.shape[0] - 1, int(cu[-1]), br,
                                            int(bool(prerotate)), int(window), _ptr(table),
                                            2 * n))
    return table


def visible_pairs(cu, window: int) -> int:
    """(query, key) pairs one head computes for this packed batch and window."""
    cu = _host_cu(cu)
    out = ctypes.c_uint64()
    _check(load_library().vlf_visible_pairs(_ptr(cu), cu.shape[0] - 1, int(cu[-1]), int(window),
                                            ctypes.byref(out)))
    return int(out.value)


def workspace_bytes(tokens: int, sequences: int, heads: int) -> int:
    """Bytes of the key-tile workspace (include/vlf.h, vlf_workspace_bytes)."""
    out = ctypes.c_int64()
    _check(load_library().vlf_workspace_bytes(int(tokens), int(sequences), int(heads),
                                              ctypes.byref(out)))
    return int(out.value)


def typical_length(cu) -> float:
    """The sequence length an average token sits in: sum(L^2) / sum(L) over the batch (0 for
    an empty batch), from the library (vlf_typical_length). Work per token grows with its
    sequence's length, so this, not the longest sequence, is what the schedule rule weighs."""
    cu = _host_cu(cu)
    out = ctypes.c_double()
    _check(load_library().vlf_typical_length(_ptr(cu), cu.shape[0] - 1, int(cu[-1]),
                                             ctypes.byref(out)))
    return float(out.value)


def schedule_rule(max_len: int, typical: float, window: int = 0, br: int = 0):
    """(br, prerotate, backward_br) from the library's rule (vlf_schedule_rule) for a batch's
    longest and typical lengths; ``br`` non-zero fixes the tile height and asks for the path."""
    b, p, bb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().vlf_schedule_rule(int(max_len), float(typical), int(window), int(br),
                                            ctypes.byref(b), ctypes.byref(p), ctypes.byref(bb)))
    return b.value, bool(p.value), bb.value


def choose_br(max_len: int, window: int = 0, typical: float | None = None) -> int:
    """Query rows per workgroup the library's rule picks (``typical`` defaults to
    ``max_len``)."""
    return schedule_rule(max_len, max_len if typical is None else typical, window)[0]


def choose_prerotate(length: float, br: int, window: int = 0, max_len: int = 0x7fffffff) -> bool:
    """Whether the library's rule takes the key-tile workspace at tile height ``br`` for a batch
    of typical length ``length`` (and longest sequence ``max_len``, unbounded by default)."""
    return schedule_rule(max_len, length, window, br)[1]


def choose_backward_br(typical: float) -> int:
    """Tile height of the backward the library's rule picks for a batch of typical length
    ``typical``."""
    return schedule_rule(0, typical)[2]


def choose_schedule(cu, heads: int, window: int = 0):
    """(br, prerotate, max_len, workspace_bytes) of the forward for this batch, from the
    library (vlf_choose_schedule)."""
    cu = _host_cu(cu)
    b, p, m, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(load_library().vlf_choose_schedule(_ptr(cu), cu.shape[0] - 1, int(cu[-1]),
                                              int(heads), int(window), ctypes.byref(b),
                                              ctypes.byref(p), ctypes.byref(m),
                                              ctypes.byref(ws)))
    return b.value, bool(p.value), m.value, int(ws.value)


def choose_backward(cu, heads: int, window: int = 0):
    """(br, workspace_bytes) of the backward for this batch, from the library
    (vlf_choose_backward)."""
    cu = _host_cu(cu)
    b, ws = ctypes.c_int32(), ctypes.c_int64()
    _check(load_library().vlf_choose_backward(_ptr(cu), cu.shape[0] - 1, int(cu[-1]),
                                              int(heads), int(window), ctypes.byref(b),
                                              ctypes.byref(ws)))
    return b.value, int(ws.value)


def forward_kernel(br: int, prerotate: bool, window: int = 0, max_len: int = 0x7fffffff) -> str:
    """Name of the forward kernel the library launches for this schedule and longest sequence
    (vlf_forward_kernel; the default max_len names the kernel for any sequence length)."""
    return load_library().vlf_forward_kernel(int(br), int(bool(prerotate)), int(window),
                                             int(max_len)).decode()


CAUSAL = 0x40000000  # ORed into a window: the causal sliding window (include/vlf.h, VLF_CAUSAL)


def window_fits_ring(window: int) -> bool:
    """Whether the direct path runs 256-row tiles under ``window`` on its LDS-resident key ring
    (the library names attend_slide for it): a tile's keys, from i0 - 64 ceil(back / 64) to
    i0 + 255 + ahead, span at most eight 64-key tiles, which holds for 1 <= W <= 129, or causal
    1 <= W <= 257."""
    return forward_kernel(256, False, window) == "attend_slide"


@dataclass
class Batch:
    """Index tensors of one packed batch on the device: cu and the tile table."""
    cu_host: np.ndarray
    cu: "torch.Tensor"
    tiles: "torch.Tensor"
    num_tiles: int
    max_len: int
    br: int
    prerotate: bool = False

    @property
    def tokens(self) -> int:
        return int(self.cu_host[-1])

    @property
    def sequences(self) -> int:
        return int(self.cu_host.shape[0] - 1)


def prepare(cu, device=None, br: int | None = None, prerotate: bool | None = None,
            window: int = 0) -> Batch:
    """Validate ``cu``, build the tile table on the host and copy both to ``device``.

    ``br`` (query rows per tile) and ``prerotate`` (use a key-tile workspace) default to the
    library's schedule rule for the longest sequence, the typical length and ``window`` (the
    window the batch will be run with; it only informs that choice)."""
    import torch
    cu_host = _host_cu(cu)
    device = torch.device("cuda") if device is None else torch.device(device)
    _, max_len = tile_count(cu_host, 128)
    rule_br, rule_pre, _ = schedule_rule(max_len, typical_length(cu_host), window,
                                         0 if br is None else int(br))
    br = rule_br
    prerotate = rule_pre if prerotate is None else bool(prerotate)
    table = launch_table(cu_host, br, prerotate, window)
    return Batch(cu_host, torch.from_numpy(cu_host).to(device),
                 torch.from_numpy(table.view(np.int32)).to(device), table.shape[0], max_len, br,
                 prerotate)


def new_workspace(batch: Batch, heads: int, device=None):
    """A uint8 device tensor sized for ``batch`` and ``heads`` (None when the batch does not
    pre-rotate)."""
    import torch
    if not batch.prerotate:
        return None
    device = batch.cu.device if device is None else torch.device(device)
    return torch.empty(workspace_bytes(batch.tokens, batch.sequences, heads),
                       dtype=torch.uint8, device=device)


_DTYPES = {}


def _dtype_code(t):
    import torch
    if not _DTYPES:
        _DTYPES.update({torch.bfloat16: VLF_BF16, torch.float16: VLF_F16})
    if t not in _DTYPES:
        raise VlfError(VLF_EUNSUPPORTED, f"dtype {t}; supported: bfloat16, float16")
    return _DTYPES[t]


def _check_inputs(batch: Batch, qkv, cos, sin, heads: int, out=None, lse=None):
    """Shapes, dtypes, contiguity and devices of the call's tensors; returns the dtype code."""
    import torch
    T = batch.tokens
    code = _dtype_code(qkv.dtype)
    checks = [("qkv", qkv, (T, 3 * heads * HEAD_DIM), qkv.dtype)]
    if out is not None:
        checks += [("out", out, (T, heads * HEAD_DIM), qkv.dtype),
                   ("lse", lse, (heads, T), torch.float32)]
    for name, t, shape, dt in checks:
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise VlfError(VLF_EINVAL, f"{name}: {tuple(t.shape)} {t.dtype} contiguous="
                                       f"{t.is_contiguous()}, expected {shape} {dt}")
    for name, t in (("cos", cos), ("sin", sin)):
        if t.dim() != 2 or t.shape[1] != HEAD_DIM // 2 or t.dtype != qkv.dtype or \
                not t.is_contiguous():
            raise VlfError(VLF_EINVAL, f"{name}: {tuple(t.shape)} {t.dtype}, expected [P, 32] "
                                       f"{qkv.dtype} contiguous")
    if cos.shape != sin.shape:
        raise VlfError(VLF_EINVAL, "cos and sin differ in shape")
    if cos.shape[0] < batch.max_len:
        raise VlfError(VLF_EINVAL, f"rotary tables have {cos.shape[0]} rows; the longest "
                                   f"sequence has {batch.max_len}")
    dev = qkv.device
    tensors = [("cos", cos), ("sin", sin), ("cu", batch.cu), ("tiles", batch.tiles)]
    if out is not None:
        tensors += [("out", out), ("lse", lse)]
    for name, t in tensors:
        if t.device != dev:
            raise VlfError(VLF_EINVAL, f"{name} is on {t.device}, qkv on {dev}")
    return code


def _workspace_args(workspace, dev):
    import torch
    if workspace is None:
        return None, 0
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or \
            workspace.device != dev:
        raise VlfError(VLF_EINVAL, f"workspace: {workspace.dtype} on {workspace.device}, "
                                   f"expected contiguous uint8 on {dev}")
    return workspace.data_ptr(), workspace.numel()


def _torch_stream(stream, dev):
    """The launch stream as a torch stream: torch's current stream of ``dev`` (None), a
    torch.cuda.Stream, or a raw hipStream_t handle."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=dev)


def _stream(stream, dev):
    return _torch_stream(stream, dev).cuda_stream


def attend_into(batch: Batch, qkv, cos, sin, heads: int, window: int, scale: float, out, lse,
                stream=None, workspace=None):
    """Queue the forward on ``stream`` (default: torch's current stream of qkv's device).

    qkv [T, 3*heads*64], cos/sin [P, 32] (same dtype, P >= longest sequence), out [T, heads*64]
    (same dtype), lse [heads, T] float32; all contiguous on one device. ``workspace``: a
    contiguous uint8 device tensor of at least ``workspace_bytes`` (from ``new_workspace``);
    when None and the batch pre-rotates, one is allocated for this call.
    """
    import torch
    code = _check_inputs(batch, qkv, cos, sin, heads, out, lse)
    dev = qkv.device
    launch = _torch_stream(stream, dev)
    if workspace is None and batch.prerotate:
        # allocated on the launch stream: when this call returns the block goes back to that
        # stream's pool, so its next user is ordered after these kernels
        with torch.cuda.stream(launch):
            workspace = new_workspace(batch, heads, dev)
    ws_ptr, ws_bytes = _workspace_args(workspace, dev)
    _check(load_library().vlf_attend(
        qkv.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0], batch.max_len,
        batch.cu.data_ptr(),
        batch.tiles.data_ptr(), batch.num_tiles, batch.br, batch.tokens, batch.sequences, heads,
        int(window), float(scale), code, ws_ptr, ws_bytes, out.data_ptr(), lse.data_ptr(),
        launch.cuda_stream))


STATIC_WORKSPACE_BYTES = 128 << 20  # include/vlf.h, VLF_STATIC_WORKSPACE_BYTES


def attend_static_into(batch: Batch, qkv, cos, sin, heads: int, window: int, scale: float, out,
                       lse, stream=None):
    """Queue the forward on the key-tile workspace path with the library's fixed device array
    as the workspace (include/vlf.h, vlf_attend_static): nothing is allocated, here or in the
    library. Batches whose workspace exceeds ``STATIC_WORKSPACE_BYTES`` are rejected; calls
    that overlap in time on one GPU race on the array."""
    code = _check_inputs(batch, qkv, cos, sin, heads, out, lse)
    dev = qkv.device
    _check(load_library().vlf_attend_static(
        qkv.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0], batch.max_len,
        batch.cu.data_ptr(), batch.tiles.data_ptr(), batch.num_tiles, batch.br, batch.tokens,
        batch.sequences, heads, int(window), float(scale), code, out.data_ptr(), lse.data_ptr(),
        _stream(stream, dev)))


def rotate_keys(batch: Batch, qkv, cos, sin, heads: int, workspace, stream=None):
    """Queue the rotation of every key tile into ``workspace`` (include/vlf.h,
    vlf_rotate_keys): the first half of ``attend_into`` with a workspace."""
    code = _check_inputs(batch, qkv, cos, sin, heads)
    dev = qkv.device
    ws_ptr, ws_bytes = _workspace_args(workspace, dev)
    _check(load_library().vlf_rotate_keys(
        qkv.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0], batch.max_len,
        batch.cu.data_ptr(),
        batch.tokens, batch.sequences, heads, code, ws_ptr, ws_bytes, _stream(stream, dev)))


def attend_rotated_into(batch: Batch, qkv, cos, sin, heads: int, window: int, scale: float,
                        out, lse, workspace, stream=None):
    """Queue the forward over a workspace ``rotate_keys`` filled for the same inputs
    (include/vlf.h, vlf_attend_rotated): the second half of ``attend_into``."""
    code = _check_inputs(batch, qkv, cos, sin, heads, out, lse)
    dev = qkv.device
    ws_ptr, ws_bytes = _workspace_args(workspace, dev)
    _check(load_library().vlf_attend_rotated(
        qkv.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0], batch.max_len,
        batch.cu.data_ptr(),
        batch.tiles.data_ptr(), batch.num_tiles, batch.br, batch.tokens, batch.sequences, heads,
        int(window), float(scale), code, ws_ptr, ws_bytes, out.data_ptr(), lse.data_ptr(),
        _stream(stream, dev)))


def rotate_qkv_into(batch: Batch, qkv, cos, sin, heads: int, scale: float, qkv_out,
                    stream=None):
    """Queue the unfused baseline's rotation pass (include/vlf.h, vlf_rotate_qkv): qkv_out gets
    the rotated, scaled queries, the rotated keys and the values, rounded as the forward rounds
    its operands."""
    code = _check_inputs(batch, qkv, cos, sin, heads)
    if tuple(qkv_out.shape) != tuple(qkv.shape) or qkv_out.dtype != qkv.dtype or \
            not qkv_out.is_contiguous() or qkv_out.device != qkv.device:
        raise VlfError(VLF_EINVAL, f"qkv_out: {tuple(qkv_out.shape)} {qkv_out.dtype}, expected "
                                   f"{tuple(qkv.shape)} {qkv.dtype} contiguous on {qkv.device}")
    dev = qkv.device
    _check(load_library().vlf_rotate_qkv(
        qkv.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0], batch.max_len,
        batch.cu.data_ptr(),
        batch.tiles.data_ptr(), batch.num_tiles, batch.br, batch.tokens, batch.sequences, heads,
        float(scale), code, qkv_out.data_ptr(), _stream(stream, dev)))


def backward_workspace_bytes(tokens: int, sequences: int, heads: int, br: int) -> int:
    """Bytes of the backward's workspace on ``br``-row tiles (per-row floats, and above 64 rows
    the 64-row tiles' operand images)."""
    n = ctypes.c_int64(0)
    _check(load_library().vlf_backward_workspace_bytes(int(tokens), int(sequences), int(heads),
                                                       int(br), ctypes.byref(n)))
    return int(n.value)


def attend_backward_into(batch: Batch, qkv, cos, sin, heads: int, window: int, scale: float,
                         out, lse, dout, dqkv, stream=None, workspace=None):
    """Queue the backward (include/vlf.h, vlf_attend_backward): dqkv = d sum(out * dout) / d qkv
    for the forward with the same arguments, whose ``out`` and ``lse`` are passed in.

    ``batch`` must be prepared with ``br`` 64, 128 or 256 (``choose_backward``). dout and dqkv
    have the shapes and dtype of out and qkv. ``workspace``: a contiguous uint8 device tensor of
    at least ``backward_workspace_bytes`` (allocated on the launch stream when None).
    """
    import torch
    if batch.br not in (64, 128, 256):
        raise VlfError(VLF_EINVAL, f"the backward runs on 64-, 128- or 256-row tiles; batch has "
                                   f"br={batch.br}")
    code = _check_inputs(batch, qkv, cos, sin, heads, out, lse)
    T = batch.tokens
    for name, t, shape in (("dout", dout, (T, heads * HEAD_DIM)),
                           ("dqkv", dqkv, (T, 3 * heads * HEAD_DIM))):
        if tuple(t.shape) != shape or t.dtype != qkv.dtype or not t.is_contiguous() or \
                t.device != qkv.device:
            raise VlfError(VLF_EINVAL, f"{name}: {tuple(t.shape)} {t.dtype} on {t.device}, "
                                       f"expected {shape} {qkv.dtype} contiguous on {qkv.device}")
    dev = qkv.device
    launch = _torch_stream(stream, dev)
    if workspace is None:
        with torch.cuda.stream(launch):
            workspace = torch.empty(backward_workspace_bytes(T, batch.sequences, heads,
                                                             batch.br),
                                    dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace_args(workspace, dev)
    _check(load_library().vlf_attend_backward(
        qkv.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0], batch.max_len,
        batch.cu.data_ptr(),
        batch.tiles.data_ptr(), batch.num_tiles, batch.br, T, batch.sequences, heads,
        int(window), float(scale), code, out.data_ptr(), dout.data_ptr(), lse.data_ptr(), ws_ptr,
        ws_bytes, dqkv.data_ptr(), launch.cuda_stream))


def attend_backward(qkv, cos, sin, cu, heads: int, out, lse, dout, window: int = 0,
                    scale: float = 0.125):
    """The backward of ``attend``: returns dqkv [T, 3*heads*64] (zero rows where no sequence
    reaches)."""
    import torch
    if isinstance(cu, Batch):
        batch = cu
    else:
        br, _ = choose_backward(cu, heads, window)
        batch = prepare(cu, qkv.device, br, False, window)
    dqkv = torch.zeros_like(qkv)
    attend_backward_into(batch, qkv, cos, sin, heads, window, scale, out, lse, dout, dqkv)
    return dqkv


def attend(qkv, cos, sin, cu, heads: int, window: int = 0, scale: float = 0.125,
           br: int | None = None, prerotate: bool | None = None):
    """Forward of packed attention; returns (out [T, heads*64], lse [heads, T] float32)."""
    import torch
    batch = cu if isinstance(cu, Batch) else prepare(cu, qkv.device, br, prerotate, window)
    T = batch.tokens
    out = torch.empty((T, heads * HEAD_DIM), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((heads, T), dtype=torch.float32, device=qkv.device)
    attend_into(batch, qkv, cos, sin, heads, window, scale, out, lse)
    return out, lse
