"""Parity of the HIP path (through the C ABI) with the float64 oracle, on the GPU.

Tolerances: max |out - oracle| <= 2e-2 for bf16 inputs and 4e-3 for fp16; max |lse - oracle|
<= 1e-3. The gate is the oracle in mode B: the query/key operands rounded to the storage type
as the subject page's kernel rounds them (hanzo-kernel 0.2.42 src/packed.rs, `attend`'s tile
loads). Every comparison also runs mode A, the unrounded definition: out must meet the same
tolerance against it too; its lse gap (the operand rounding alone moves the scores by more than
1e-3 in bf16) is printed.

Every case compares every output row, the full-size encoder, sliding-window and many-short
workloads included, which run exactly as bench.py launches them. The long workload (131072
rows) compares two rows of every 32-row wave block of every query tile, all heads, so every
workgroup and every wave of its launch is checked, plus properties of all rows. Guard regions
after `out` and `lse` must stay untouched.
"""
import functools
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import variable_length_flash_amd as vlf
from variable_length_flash_amd import workloads

pytestmark = pytest.mark.gpu

OUT_TOL = {"bf16": 2e-2, "fp16": 4e-3}
LSE_TOL = 1e-3
GUARD = 4096


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, qkv, cos, sin, br=None, window=None, prerotate=None, workspace=None):
    """The HIP path on cuda:0 with NaN-filled outputs and guard regions; returns numpy arrays.
    ``prerotate`` picks the path (None: the binding's default for the batch)."""
    window = w.window if window is None else window
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev, br, prerotate, window)
    q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
    T, H = w.tokens, w.heads
    out_buf = torch.full((T * H * 64 + GUARD,), float("nan"), dtype=qkv.dtype, device=dev)
    lse_buf = torch.full((H * T + GUARD,), float("nan"), dtype=torch.float32, device=dev)
    out = out_buf[:T * H * 64].view(T, H * 64)
    lse = lse_buf[:H * T].view(H, T)
    vlf.attend_into(batch, q, c, s, H, window, w.scale, out, lse, workspace=workspace)
    torch.cuda.synchronize()
    assert torch.isnan(out_buf[T * H * 64:]).all(), "out guard region was written"
    assert torch.isnan(lse_buf[H * T:]).all(), "lse guard region was written"
    return out.float().cpu().numpy(), lse.cpu().numpy()


def inputs(w):
    qkv = workloads.draw_qkv(w)
    cos, sin = workloads.rope_tables(w)
    return qkv, cos, sin


def compare(name, w, got_out, got_lse, qkv, cos, sin, rows=None, window=None, mode_a=True):
    """The gate: out and lse against the mode-B oracle; out also against mode A unless
    ``mode_a`` is False (inputs far from the workloads' N(0, 1) recipe, where rounding the
    operands alone moves the oracle's own out by more than the tolerance)."""
    window = w.window if window is None else window
    q32 = qkv.float().numpy()
    c32, s32 = cos.float().numpy(), sin.float().numpy()
    want_out, want_lse = oracle.attend(q32, c32, s32, w.cu, w.heads, window, w.scale, mode="B",
                                       dtype=w.dtype, rows=rows)
    a_out, a_lse = oracle.attend(q32, c32, s32, w.cu, w.heads, window, w.scale, mode="A",
                                 dtype=w.dtype, rows=rows)
    if rows is not None:
        got_out, got_lse = got_out[rows], got_lse[:, rows]
    assert np.isfinite(got_out).all() and np.isfinite(got_lse).all(), "unwritten or non-finite"
    e_out = float(np.abs(got_out - want_out).max()) if got_out.size else 0.0
    e_lse = float(np.abs(got_lse - want_lse).max()) if got_lse.size else 0.0
    a_eo = float(np.abs(got_out - a_out).max()) if got_out.size else 0.0
    a_el = float(np.abs(got_lse - a_lse).max()) if got_lse.size else 0.0
    _say(f"[parity] {name}: out {e_out:.2e} (tol {OUT_TOL[w.dtype]:.0e}), lse {e_lse:.2e} "
         f"(tol {LSE_TOL:.0e}); vs unrounded definition: out {a_eo:.2e}, lse {a_el:.2e}")
    assert e_out <= OUT_TOL[w.dtype], (name, e_out)
    assert e_lse <= LSE_TOL, (name, e_lse)
    if mode_a:
        assert a_eo <= OUT_TOL[w.dtype], (name, "out against mode A", a_eo)


LENS = [5, 40, 1, 33, 70]


PATHS = [False, True]  # prerotate: every workgroup rotates its key tiles / key-tile workspace


@pytest.mark.parametrize("prerotate", PATHS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("br", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 9, 65])
def test_page_fixture(dtype, br, window, prerotate):
    w = workloads.custom(LENS, 2, dtype=dtype, window=window, table_rows=128, seed=7)
    qkv, cos, sin = inputs(w)
    _say(f"case page-fixture {dtype} br={br} W={window} prerotate={prerotate}")
    out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=prerotate)
    compare(f"lens {LENS} {dtype} br={br} W={window} pre={int(prerotate)}", w, out, lse, qkv,
            cos, sin)


def test_tiny_workload():
    w = workloads.tiny()
    qkv, cos, sin = inputs(w)
    _say("case tiny")
    out, lse = run_gpu(w, qkv, cos, sin)
    compare("tiny", w, out, lse, qkv, cos, sin)


RAGGED = [1, 63, 64, 65, 127, 128, 129, 300, 0, 257, 31, 32, 33, 2]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", [0, 1, 2, 31, 32, 33, 64, 65, 128, 200, 1000])
def test_ragged_tiles_and_windows(dtype, window):
    w = workloads.custom(RAGGED, 3, dtype=dtype, window=window, base=1e4, table_rows=512,
                         seed=11)
    qkv, cos, sin = inputs(w)
    for br in (64, 128, 256):
        for pre in PATHS:
            _say(f"case ragged {dtype} W={window} br={br} prerotate={pre}")
            out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=pre)
            compare(f"ragged {dtype} W={window} br={br} pre={int(pre)}", w, out, lse, qkv, cos,
                    sin)


@pytest.mark.parametrize("prerotate", PATHS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("br", [64, 128, 256])
def test_single_key_rows_are_exact(dtype, br, prerotate):
    """W = 1: each row sees only itself, so out = v (bit-exact) and lse = <q~, k~>, one float32
    dot product of the rounded operands. Agreement with the oracle's float64 dot product of its
    own rounded operands to float32 accumulation error (far below one storage-type ulp of a
    single operand) shows the kernel's rotated, scaled and rounded operands are the oracle's."""
    w = workloads.custom([1, 7, 130, 64, 300], 2, dtype=dtype, window=1, table_rows=512, seed=5)
    qkv, cos, sin = inputs(w)
    _say(f"case single-key {dtype} br={br} prerotate={prerotate}")
    out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=prerotate)
    hd = w.heads * 64
    np.testing.assert_array_equal(out, qkv[:, 2 * hd:].float().numpy())
    _, want = oracle.attend(qkv.float().numpy(), cos.float().numpy(), sin.float().numpy(), w.cu,
                            w.heads, 1, w.scale, mode="B", dtype=dtype)
    err = float(np.abs(lse - want).max())
    _say(f"[parity] single-key rows {dtype} br={br}: lse {err:.2e} (tol 2e-5)")
    assert err < 2e-5


@pytest.mark.parametrize("prerotate", PATHS)
@pytest.mark.parametrize("lens", [[1], [1] * 300, [0, 0, 5, 0], [64] * 9, [128, 1, 128],
                                  [2048], [0, 777, 0, 0, 1500], [3] * 700 + [300],
                                  [0] * 400 + [70] + [0] * 200 + [1]])
def test_edge_batches(lens, prerotate):
    w = workloads.custom(lens, 2, dtype="fp16", window=0, table_rows=max(lens + [1]), seed=3)
    qkv, cos, sin = inputs(w)
    _say(f"case edge {lens[:6]} prerotate={prerotate}")
    out, lse = run_gpu(w, qkv, cos, sin, prerotate=prerotate)
    compare(f"edge {lens[:6]}{'...' if len(lens) > 6 else ''} pre={int(prerotate)}", w, out,
            lse, qkv, cos, sin)


@pytest.mark.parametrize("name,br,window", [("ragged", 64, 0), ("ragged", 128, 33),
                                            ("ragged", 256, 200), ("encoder", 128, 0),
                                            ("sliding", 256, 128), ("long", 256, 0)])
def test_paths_agree(name, br, window):
    """Both paths stage the same rounded operands and run the same products. They keep
    different reference maxima (the workspace path fixes each row's reference from a norm
    bound before its key loop), so the probabilities are rounded at different scales: lse, from
    the same unrounded sums, agrees to float32 rounding; out to about one bf16 ulp."""
    if name == "ragged":
        w = workloads.custom(RAGGED, 3, dtype="bf16", window=window, table_rows=512, seed=13)
    else:
        w = workloads.WORKLOADS[name]()
    qkv, cos, sin = inputs(w)
    _say(f"case paths agree {name} br={br} W={window}")
    a_out, a_lse = run_gpu(w, qkv, cos, sin, br=br, window=window, prerotate=False)
    b_out, b_lse = run_gpu(w, qkv, cos, sin, br=br, window=window, prerotate=True)
    d_out = float(np.abs(a_out - b_out).max()) if a_out.size else 0.0
    d_lse = float(np.abs(a_lse - b_lse).max()) if a_lse.size else 0.0
    _say(f"[paths] {name} br={br} W={window}: out {d_out:.2e}, lse {d_lse:.2e}")
    assert d_lse <= 2e-5 and d_out <= 8e-3, (d_out, d_lse)


def test_workspace_is_rewritten_on_every_call():
    """A reused workspace (filled with NaN bit patterns, then reused by a smaller batch) gives
    the same result as a fresh one: every block a tile reads is written in the same call."""
    dev = torch.device("cuda:0")
    big = workloads.custom([700, 1300, 64], 2, dtype="bf16", window=0, table_rows=2048, seed=21)
    small = workloads.custom([300, 65, 1], 2, dtype="bf16", window=0, table_rows=2048, seed=22)
    ws = torch.full((vlf.workspace_bytes(big.tokens, big.sequences, big.heads),), 0xFF,
                    dtype=torch.uint8, device=dev)
    for w in (big, small):
        qkv, cos, sin = inputs(w)
        _say(f"case workspace reuse T={w.tokens}")
        out, lse = run_gpu(w, qkv, cos, sin, prerotate=True, workspace=ws)
        compare(f"workspace reuse T={w.tokens}", w, out, lse, qkv, cos, sin)


def test_empty_batch_launches_nothing():
    w = workloads.custom([0, 0], 2, dtype="bf16", table_rows=4)
    qkv, cos, sin = inputs(w)
    out, lse = run_gpu(w, qkv, cos, sin)
    assert out.shape == (0, 128) and lse.shape == (2, 0)


def test_stream_and_repeat_are_deterministic():
    """Two launches on a side stream give identical bits."""
    w = workloads.custom([300, 41, 999], 4, dtype="bf16", window=0, table_rows=1024, seed=9)
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev)
    q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
    side = torch.cuda.Stream(dev)
    outs = []
    with torch.cuda.stream(side):
        for _ in range(2):
            o = torch.empty((w.tokens, w.heads * 64), dtype=qkv.dtype, device=dev)
            l = torch.empty((w.heads, w.tokens), dtype=torch.float32, device=dev)
            vlf.attend_into(batch, q, c, s, w.heads, 0, w.scale, o, l)
            outs.append((o, l))
    side.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_explicit_stream_keeps_its_workspace():
    """A launch on an explicit stream (torch stream or raw handle) while another stream is
    current: the workspace the binding allocates belongs to the launch stream, so an allocation
    of the same size made right after on the current stream, and overwritten there, cannot be
    handed that memory while the kernels still read it."""
    w = workloads.custom([300, 41, 999], 4, dtype="bf16", window=0, table_rows=1024, seed=9)
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev)
    assert batch.prerotate
    q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
    nbytes = vlf.workspace_bytes(w.tokens, w.sequences, w.heads)
    ref_o = torch.empty((w.tokens, w.heads * 64), dtype=qkv.dtype, device=dev)
    ref_l = torch.empty((w.heads, w.tokens), dtype=torch.float32, device=dev)
    vlf.attend_into(batch, q, c, s, w.heads, 0, w.scale, ref_o, ref_l)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    for handle in (side, side.cuda_stream):
        o = torch.empty_like(ref_o)
        l = torch.empty_like(ref_l)
        side.wait_stream(torch.cuda.current_stream(dev))
        vlf.attend_into(batch, q, c, s, w.heads, 0, w.scale, o, l, stream=handle)
        clobber = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        clobber.fill_(0xFF)
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"stream={type(handle)}"


def sample_rows(w, br, count, seed):
    """For the stress cases below (not the five workloads): first / last rows of every
    sequence, rows at tile and wave boundaries of a spread of tiles, and random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    cu = w.cu
    for s in range(w.sequences):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            rows.update([a, b - 1])
    tiles = vlf.tile_table(cu, br)
    pick = tiles[rng.choice(len(tiles), size=min(len(tiles), 64), replace=False)]
    for s, i0 in pick:
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for off in (0, 31, 32, 63, 64, 95, 96, br - 1):
            if i0 + off < L:
                rows.add(a + int(i0) + off)
    extra = max(0, count - len(rows))
    rows.update(rng.integers(0, w.tokens, size=extra).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def wave_block_rows(w, br):
    """Two rows of every 32-row wave block of every ``br``-row query tile (offsets that cycle
    through all 32 lanes of a block from one block to the next), plus every sequence's first
    and last rows: every workgroup and every wave of the launch computes some of them."""
    rows = set()
    cu = w.cu
    k = 0
    for s in range(w.sequences):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        if L == 0:
            continue
        rows.update([a, a + L - 1])
        for b0 in range(0, L, 32):
            for off in ((11 * k) % 32, (11 * k + 16) % 32):
                if b0 + off < L:
                    rows.add(a + b0 + off)
            k += 1
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["encoder", "sliding", "many_short", "long"])
def test_full_size_workload(name):
    w = workloads.WORKLOADS[name]()
    _say(f"case full-size {name}: T={w.tokens} S={w.sequences} H={w.heads} {w.dtype} "
         f"W={w.window}")
    qkv, cos, sin = inputs(w)
    out, lse = run_gpu(w, qkv, cos, sin)
    # every row written and finite; each out row lies within the span of the visible values
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    vmax = float(qkv[:, 2 * w.heads * 64:].float().abs().max())
    assert np.abs(out).max() <= vmax * (1 + 2 ** -7)
    if name != "long":
        compare(f"{name} (all {w.tokens} rows, all heads)", w, out, lse, qkv, cos, sin)
        return
    br = vlf.choose_br(max(w.lens), w.window, vlf.typical_length(w.cu))
    rows = wave_block_rows(w, br)
    assert len(rows) >= 2 * w.tokens // 32
    compare(f"{name} ({len(rows)} rows: two of every 32-row wave block, all heads)", w, out, lse,
            qkv, cos, sin, rows=rows)


@functools.lru_cache(maxsize=1)
def _tie_inputs(seed=31, length=64):
    """fp16 inputs whose key rotations land exactly on binary16 ties after the float32
    rounding the page prescribes (float32 fma, then the cast), while the exact value is off the
    tie: a fused fma-and-narrow would round those keys the other way. One head, one sequence;
    queries and values random. Returns (qkv [L, 192] float16, cos, sin [L, 32] float16)."""
    rng = np.random.default_rng(seed)
    need = length * 32
    found = []
    while sum(len(f[0]) for f in found) < need:
        n = 1 << 21
        x1 = rng.standard_normal(n).astype(np.float16).astype(np.float64)
        x2 = rng.standard_normal(n).astype(np.float16).astype(np.float64)
        c = rng.uniform(-1, 1, n).astype(np.float16).astype(np.float64)
        s = rng.uniform(-1, 1, n).astype(np.float16).astype(np.float64)
        exact = x1 * c - x2 * s               # exact: products of binary16 values fit float64
        y = exact.astype(np.float32)
        bits = y.view(np.uint32)
        normal = (np.abs(y) >= 2.0 ** -14) & (np.abs(y) < 60000)
        tie = normal & ((bits & 0x1FFF) == 0x1000) & (exact != y.astype(np.float64))
        k = np.nonzero(tie)[0]
        found.append((x1[k], x2[k], c[k], s[k]))
    x1, x2, c, s = (np.concatenate([f[i] for f in found])[:need].reshape(length, 32)
                    for i in range(4))
    qkv = np.zeros((length, 3 * 64), dtype=np.float16)
    qkv[:, :64] = rng.standard_normal((length, 64)).astype(np.float16)
    qkv[:, 64:96] = x1
    qkv[:, 96:128] = x2
    qkv[:, 128:] = rng.standard_normal((length, 64)).astype(np.float16)
    return (torch.from_numpy(qkv), torch.from_numpy(c.astype(np.float16)),
            torch.from_numpy(s.astype(np.float16)))


@pytest.mark.parametrize("prerotate", PATHS)
@pytest.mark.parametrize("br", [64, 128, 256])
def test_key_rotation_ties_round_like_the_page(br, prerotate):
    """Every key element sits on a binary16 tie after its float32 rounding. With W = 1 each row
    sees only itself: out = v bit for bit and lse = <q~, k~> to float32 accumulation error, so
    a key rounded the other way (about one binary16 ulp times |q~|, ~1e-4) cannot pass."""
    qkv, cos, sin = _tie_inputs()
    w = workloads.custom([64], 1, dtype="fp16", window=1, table_rows=64, seed=0)
    _say(f"case key ties br={br} prerotate={prerotate}")
    out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=prerotate)
    np.testing.assert_array_equal(out, qkv[:, 128:].float().numpy())
    _, want = oracle.attend(qkv.float().numpy(), cos.float().numpy(), sin.float().numpy(), w.cu,
                            1, 1, w.scale, mode="B", dtype="fp16")
    err = float(np.abs(lse - want).max())
    _say(f"[parity] key ties br={br} pre={int(prerotate)}: lse {err:.2e} (tol 2e-5)")
    assert err < 2e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("factor", [6.0, 12.0])
@pytest.mark.parametrize("window", [0, 300])
def test_outlying_key_norms(dtype, factor, window):
    """A few keys scaled far beyond the rest loosen the norm bound of every score in their
    tiles' sweeps. With the factor 6 a bfloat16 row's reference on the 256-row workspace path
    can sit some 30 above its largest score (probabilities near e^-30); with 12, and for every
    fp16 row whose bound is loose, the kernel first sweeps the scores for the exact row
    maximum. Every row must match the oracle on both paths and at every tile height. Mode A is
    printed, not gated: with keys scaled by 6 or 12 the oracle's own mode-B out lies 4.8e-2 to
    9.6e-2 (bf16) and 4.8e-3 to 9.4e-3 (fp16) from mode A, so no kernel that rounds its operands
    to the storage type can be within the out tolerance of the unrounded definition."""
    w = workloads.custom([700, 300, 65], 2, dtype=dtype, window=window, table_rows=1024,
                         seed=41)
    qkv, cos, sin = inputs(w)
    x = qkv.float()
    H = w.heads
    for t in (3, 350, 699, 830, 1007):
        x[t, H * 64:2 * H * 64] *= factor
    qkv = x.to(qkv.dtype)
    for br in (64, 128, 256):
        for pre in PATHS:
            _say(f"case outlying keys {dtype} x{factor} W={window} br={br} prerotate={pre}")
            out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=pre)
            compare(f"outlying keys {dtype} x{factor} W={window} br={br} pre={int(pre)}", w,
                    out, lse, qkv, cos, sin, mode_a=False)


@functools.lru_cache(maxsize=1)
def _wide_inputs():
    """88 sequences of 1024 tokens, 64 heads, bf16, tables of 90112 rows: qkv spans 2.2 GB, so
    byte offsets from its start pass 2^31 and the direct path builds a buffer descriptor per
    key tile instead of one per sequence (its whole-sequence form needs every offset below
    2^31)."""
    w = workloads.custom([1024] * 88, 64, dtype="bf16", window=0, base=1.6e5, table_rows=90112,
                         seed=23)
    qkv, cos, sin = inputs(w)
    return w, qkv, cos, sin


@pytest.mark.parametrize("window", [0, 128, 300])
def test_offsets_past_2gib(window):
    """Rows past 2^31 bytes from the first: per-tile descriptors on the direct path (W = 128 at
    256 rows is the key ring's, with about 88 items per workgroup, so its item descriptors are
    refilled mid-run), 64-bit offsets on the workspace path."""
    w, qkv, cos, sin = _wide_inputs()
    assert qkv.numel() * 2 > 2 ** 31
    w_rows = sample_rows(w, 128, 1200, seed=9)
    assert w_rows[-1] == w.tokens - 1
    for br, pre in ((64, False), (128, False), (256, False), (256, True)):
        _say(f"case offsets past 2 GiB W={window} br={br} prerotate={pre}")
        out, lse = run_gpu(w, qkv, cos, sin, br=br, window=window, prerotate=pre)
        compare(f"qkv of 2.2 GB W={window} br={br} pre={int(pre)} ({len(w_rows)} rows)", w, out,
                lse, qkv, cos, sin, rows=w_rows, window=window)


@pytest.mark.parametrize("window", [0, 1000])
def test_fp16_long_sequences_on_the_workspace_path(window):
    """Two sequences of 8192 tokens in fp16 on the workspace path. Its fixed reference may sit
    no higher than a row's largest score for binary16, so with N(0, 1) inputs a share of waves
    takes the exact-maximum sweep; sampled rows against the oracle."""
    w = workloads.custom([8192, 8192], 4, dtype="fp16", window=window, base=1.6e5,
                         table_rows=8192, seed=29)
    qkv, cos, sin = inputs(w)
    rows = sample_rows(w, 256, 900, seed=17)
    for br in (128, 256):
        _say(f"case fp16 long workspace W={window} br={br}")
        out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=True)
        compare(f"fp16 2 x 8192 W={window} br={br} pre=1 ({len(rows)} rows)", w, out, lse, qkv,
                cos, sin, rows=rows)


RUN_LENS = [9000, 0, 7001, 1, 300, 5000, 129, 64, 65]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", [1, 64, 127, 128, 129])
def test_window_runs_keep_keys(dtype, window):
    """Direct path, 256-row tiles, windows of at most 129 keys: one workgroup per CU walks a run
    of (head, tile) items and keeps the window's key tiles in LDS from one item to the next.
    1408 items, so every run spans several and crosses sequences (an empty one, one-row and
    one-tile ones) and heads."""
    w = workloads.custom(RUN_LENS, 16, dtype=dtype, window=window, base=1.6e5, table_rows=9000,
                         seed=43)
    qkv, cos, sin = inputs(w)
    _say(f"case window runs {dtype} W={window}")
    out, lse = run_gpu(w, qkv, cos, sin, br=256, prerotate=False)
    compare(f"window runs {dtype} W={window}", w, out, lse, qkv, cos, sin)


# sequences of at most 512 tokens: every length class around the eight-tile ring's edges
WHOLE_LENS = [512, 1, 0, 63, 64, 65, 255, 256, 257, 511, 300, 512, 129, 2, 448, 77] * 6


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", [0, 1, 100, 130, 300, 600, 0 | vlf.CAUSAL, 200 | vlf.CAUSAL])
def test_whole_sequences_in_the_key_ring(dtype, window):
    """No sequence longer than 512 tokens: the direct path at 256 rows keeps each (sequence,
    head)'s whole key range in attend_slide's eight-tile ring, under any window (wider ones
    than the ring's window bound included). The library names attend_slide for the batch;
    every row of 96 sequences x 12 heads is compared."""
    w = workloads.custom(WHOLE_LENS, 12, dtype=dtype, window=window, table_rows=512, seed=59)
    assert vlf.forward_kernel(256, False, window, max(w.lens)) == "attend_slide"
    qkv, cos, sin = inputs(w)
    _say(f"case whole sequences in the key ring {dtype} W={window:#x}")
    out, lse = run_gpu(w, qkv, cos, sin, br=256, prerotate=False)
    compare(f"whole sequences in the ring {dtype} W={window:#x}", w, out, lse, qkv, cos, sin)


def test_understated_max_len_skips_what_the_ring_cannot_hold():
    """max_len also picks the kernel, and the library cannot check it against cu on the device:
    told 512 for a batch whose middle sequence has 1000 tokens (tables long enough for it), the
    direct path at 256 rows runs the ring kernel, which must skip that sequence's tiles (their
    keys span 16 key tiles) and leave its rows unwritten, while the other sequences are exact."""
    import dataclasses
    lens = [300, 1000, 64]
    w = workloads.custom(lens, 2, dtype="bf16", window=0, table_rows=1000, seed=61)
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev, 256, False, 0)
    assert batch.max_len == 1000
    batch = dataclasses.replace(batch, max_len=512)
    assert vlf.forward_kernel(256, False, 0, batch.max_len) == "attend_slide"
    T, H = w.tokens, w.heads
    out = torch.full((T, H * 64), float("nan"), dtype=qkv.dtype, device=dev)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev)
    _say("case understated max_len on the key ring")
    vlf.attend_into(batch, qkv.to(dev), cos.to(dev), sin.to(dev), H, 0, w.scale, out, lse)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    skipped = np.arange(300, 1300)
    assert np.isnan(out[skipped]).all() and np.isnan(lse[:, skipped]).all()
    kept = np.r_[np.arange(0, 300), np.arange(1300, 1364)]
    compare("understated max_len: the sequences the ring holds", w, out, lse, qkv, cos, sin,
            rows=kept)


# 80 sequences of 0 to 512 tokens x 8 heads: 640 (sequence, head) runs, at least two for each
# of a 256-CU device's workgroups, so attend_slide deals whole runs in snake order
SNAKE_LENS = [int(x) for x in np.random.default_rng(71).integers(0, 513, size=80)]
SNAKE_LENS[5] = SNAKE_LENS[40] = 0
SNAKE_LENS[6], SNAKE_LENS[7] = 1, 512


def _with_table(batch, table, dev):
    import dataclasses
    tiles = torch.from_numpy(np.ascontiguousarray(table).astype(np.uint32).view(np.int32))
    return dataclasses.replace(batch, tiles=tiles.to(dev).contiguous(), num_tiles=len(table))


def _attend_nan(batch, w, qkv, cos, sin, dev):
    T, H = w.tokens, w.heads
    out = torch.full((T, H * 64), float("nan"), dtype=qkv.dtype, device=dev)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev)
    vlf.attend_into(batch, qkv.to(dev), cos.to(dev), sin.to(dev), H, w.window, w.scale, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def test_snake_order_ignores_the_table_order():
    """With at least two whole (sequence, head) runs per workgroup and at most 256 sequences,
    attend_slide ranks the sequences by cost from cu and deals the runs in snake order, so the
    table's order does not matter: the canonical, reversed, shuffled and doubled tables give
    bit-identical outputs, and the canonical one matches the oracle on every row."""
    w = workloads.custom(SNAKE_LENS, 8, dtype="bf16", window=0, table_rows=512, seed=73)
    assert vlf.forward_kernel(256, False, 0, max(w.lens)) == "attend_slide"
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev, 256, False, 0)
    canon = vlf.tile_table(w.cu, 256).astype(np.int64)
    _say("case snake order, canonical table")
    ref = _attend_nan(_with_table(batch, canon, dev), w, qkv, cos, sin, dev)
    compare("snake order, canonical table", w, ref[0], ref[1], qkv, cos, sin)
    rng = np.random.default_rng(9)
    for name, table in (("reversed", canon[::-1]), ("shuffled", canon[rng.permutation(len(canon))]),
                        ("doubled", np.repeat(canon, 2, axis=0))):
        _say(f"case snake order, {name} table")
        got = _attend_nan(_with_table(batch, table, dev), w, qkv, cos, sin, dev)
        assert np.array_equal(got[0], ref[0], equal_nan=True), name
        assert np.array_equal(got[1], ref[1], equal_nan=True), name


@pytest.mark.parametrize("count", [256, 257])
def test_snake_order_at_its_sequence_bound(count):
    """256 sequences is the most attend_slide ranks itself (snake order); 257 take equal runs of
    the table. Both exact on every row, 2 heads, sequences of 0 to 300 tokens."""
    lens = [int(x) for x in np.random.default_rng(count).integers(0, 301, size=count)]
    w = workloads.custom(lens, 2, dtype="fp16", window=0, table_rows=300, seed=count)
    qkv, cos, sin = inputs(w)
    _say(f"case snake order bound, {count} sequences")
    out, lse = run_gpu(w, qkv, cos, sin, br=256, prerotate=False)
    compare(f"{count} sequences on the key ring", w, out, lse, qkv, cos, sin)


def test_understated_max_len_in_snake_order():
    """Snake order ranks only the sequences the tables reach: told max_len 300 (tables of 300
    rows) for a batch with a 600-token sequence among 100 short ones, the ring kernel leaves the
    long sequence's rows unwritten and the others exact (the oracle, which wants tables for
    every sequence, gets 600 rows whose first 300 are the kernel's)."""
    import dataclasses
    lens = [int(x) for x in np.random.default_rng(75).integers(1, 201, size=100)]
    lens[50] = 600
    w = workloads.custom(lens, 8, dtype="bf16", window=0, table_rows=300, seed=75)
    qkv, cos, sin = inputs(w)
    w_full = workloads.custom(lens, 8, dtype="bf16", window=0, table_rows=600, seed=75)
    cos_full, sin_full = workloads.rope_tables(w_full)
    assert torch.equal(cos_full[:300], cos) and torch.equal(sin_full[:300], sin)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev, 256, False, 0)
    batch = dataclasses.replace(batch, max_len=300)
    assert vlf.forward_kernel(256, False, 0, batch.max_len) == "attend_slide"
    _say("case understated max_len in snake order")
    out, lse = _attend_nan(batch, w, qkv, cos, sin, dev)
    a, b = int(w.cu[50]), int(w.cu[51])
    assert np.isnan(out[a:b]).all() and np.isnan(lse[:, a:b]).all()
    kept = np.r_[np.arange(0, a), np.arange(b, w.tokens)]
    compare("understated max_len in snake order", w_full, out, lse, qkv, cos_full, sin_full,
            rows=kept)


def test_understated_max_len_on_single_key_tile_rows():
    """At 64 rows a max_len of at most 64 runs attend_one's single-tile form, which sweeps one
    key tile: told 64 for a batch with a 100-token sequence (tables long enough for it), that
    sequence's two query tiles reach two key tiles and must be left unwritten, while the
    sequences of at most 64 tokens are exact."""
    import dataclasses
    lens = [40, 100, 64, 1]
    w = workloads.custom(lens, 2, dtype="fp16", window=0, table_rows=100, seed=62)
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = dataclasses.replace(vlf.prepare(w.cu, dev, 64, False, 0), max_len=64)
    T, H = w.tokens, w.heads
    out = torch.full((T, H * 64), float("nan"), dtype=qkv.dtype, device=dev)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev)
    _say("case understated max_len on single-tile rows")
    vlf.attend_into(batch, qkv.to(dev), cos.to(dev), sin.to(dev), H, 0, w.scale, out, lse)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    skipped = np.arange(40, 140)
    assert np.isnan(out[skipped]).all() and np.isnan(lse[:, skipped]).all()
    kept = np.r_[np.arange(0, 40), np.arange(140, 205)]
    compare("understated max_len: the single-tile sequences", w, out, lse, qkv, cos, sin,
            rows=kept)


@pytest.mark.parametrize("window", [1, 65])
def test_window_runs_past_the_descriptor_cache(window):
    """20000 one-token sequences among longer ones, 2 heads: about 160 items per workgroup of
    the key ring, so each run refills its LDS item descriptors (64 at a time) two or three
    times, and most items start a new sequence on a cold ring."""
    lens = [1] * 20000
    for k, L in ((3, 700), (5000, 300), (12000, 257), (19999, 1000)):
        lens[k] = L
    w = workloads.custom(lens, 2, dtype="bf16", window=window, table_rows=1000, seed=53)
    qkv, cos, sin = inputs(w)
    _say(f"case window runs past the descriptor cache W={window}")
    out, lse = run_gpu(w, qkv, cos, sin, br=256, prerotate=False)
    compare(f"20000 one-token sequences W={window}", w, out, lse, qkv, cos, sin)


@pytest.mark.parametrize("order", ["shuffled", "reversed", "doubled"])
def test_window_runs_in_any_table_order(order):
    """The kept key tiles follow the table order: a shuffled table (with entries that name no
    tile), a reversed one and one that lists every tile twice in a row give the canonical
    results."""
    import dataclasses
    lens = [3000, 0, 77, 2000, 1, 129, 700]
    w = workloads.custom(lens, 24, dtype="bf16", window=100, table_rows=3000, seed=47)
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev, 256, False, w.window)
    canon = vlf.tile_table(w.cu, 256).astype(np.int64)
    if order == "shuffled":
        foreign = np.array([[len(lens), 0], [0, 3000], [2, 77], [4, 2 ** 32 - 1], [1, 0]],
                           dtype=np.int64)
        table = np.concatenate([canon, foreign])
        table = table[np.random.default_rng(5).permutation(len(table))]
    elif order == "reversed":
        table = canon[::-1]
    else:
        table = np.repeat(canon, 2, axis=0)
    tiles = torch.from_numpy(np.ascontiguousarray(table).astype(np.uint32).view(np.int32))
    batch = dataclasses.replace(batch, tiles=tiles.to(dev).contiguous(), num_tiles=len(table))
    T, H = w.tokens, w.heads
    out_buf = torch.full((T * H * 64 + GUARD,), float("nan"), dtype=qkv.dtype, device=dev)
    lse_buf = torch.full((H * T + GUARD,), float("nan"), dtype=torch.float32, device=dev)
    out = out_buf[:T * H * 64].view(T, H * 64)
    lse = lse_buf[:H * T].view(H, T)
    _say(f"case window runs, {order} table")
    vlf.attend_into(batch, qkv.to(dev), cos.to(dev), sin.to(dev), H, w.window, w.scale, out,
                    lse)
    torch.cuda.synchronize()
    assert torch.isnan(out_buf[T * H * 64:]).all() and torch.isnan(lse_buf[H * T:]).all()
    compare(f"window runs, {order} table", w, out.float().cpu().numpy(), lse.cpu().numpy(),
            qkv, cos, sin)


@pytest.mark.parametrize("prerotate", PATHS)
@pytest.mark.parametrize("br", [64, 128, 256])
def test_tile_order_and_foreign_entries(br, prerotate):
    """The tile table is the launch order and may be any permutation of the canonical one; its
    entries naming a sequence past S or a first row at or past the sequence end (including
    2^32 - 1, read as -1) are skipped without writing anything."""
    import dataclasses
    lens = [300, 0, 77, 513, 1, 129]
    w = workloads.custom(lens, 3, dtype="bf16", window=0, table_rows=600, seed=37)
    qkv, cos, sin = inputs(w)
    dev = torch.device("cuda:0")
    batch = vlf.prepare(w.cu, dev, br, prerotate, 0)
    canon = vlf.tile_table(w.cu, br).astype(np.int64)
    rng = np.random.default_rng(br + 7 * int(prerotate))
    foreign = np.array([[len(lens), 0], [len(lens) + 5, 0], [0, 300], [0, 300 + 64],
                        [2, 77], [4, 2 ** 32 - 1], [1, 0]], dtype=np.int64)
    table = np.concatenate([canon, foreign])[rng.permutation(len(canon) + len(foreign))]
    tiles = torch.from_numpy(table.astype(np.uint32).view(np.int32)).to(dev).contiguous()
    batch = dataclasses.replace(batch, tiles=tiles, num_tiles=len(table))
    T, H = w.tokens, w.heads
    out_buf = torch.full((T * H * 64 + GUARD,), float("nan"), dtype=qkv.dtype, device=dev)
    lse_buf = torch.full((H * T + GUARD,), float("nan"), dtype=torch.float32, device=dev)
    out = out_buf[:T * H * 64].view(T, H * 64)
    lse = lse_buf[:H * T].view(H, T)
    _say(f"case shuffled table br={br} prerotate={prerotate}")
    vlf.attend_into(batch, qkv.to(dev), cos.to(dev), sin.to(dev), H, 0, w.scale, out, lse)
    torch.cuda.synchronize()
    assert torch.isnan(out_buf[T * H * 64:]).all() and torch.isnan(lse_buf[H * T:]).all()
    compare(f"shuffled table with foreign entries br={br} pre={int(prerotate)}", w,
            out.float().cpu().numpy(), lse.cpu().numpy(), qkv, cos, sin)


# ---- the causal sliding window (window | CAUSAL): keys i - W < j <= i, or j <= i for W = 0

CAUSAL_LENS = [5, 40, 1, 33, 70, 0, 300, 257, 64, 65, 1000]


@pytest.mark.parametrize("prerotate", PATHS)
@pytest.mark.parametrize("br", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 1, 9, 65, 200])
def test_causal_window(window, br, prerotate):
    """Every kernel of both paths under the causal mask, bf16, on ragged sequences up to 1000
    tokens (several key tiles behind each query tile, none ahead); every output row."""
    w = workloads.custom(CAUSAL_LENS, 2, dtype="bf16", window=window | vlf.CAUSAL, base=1.6e5,
                         table_rows=1000, seed=37)
    qkv, cos, sin = inputs(w)
    _say(f"case causal W={window} br={br} prerotate={prerotate}")
    out, lse = run_gpu(w, qkv, cos, sin, br=br, prerotate=prerotate)
    compare(f"causal W={window} br={br} pre={int(prerotate)}", w, out, lse, qkv, cos, sin)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", [1, 64, 129, 200, 257])
def test_causal_window_runs_keep_keys(dtype, window):
    """The key ring (attend_slide) under causal windows: nothing ahead of a query tile, so
    windows up to 257 keys fit its eight tiles. Runs of items across sequences and heads."""
    assert vlf.binding.window_fits_ring(window | vlf.CAUSAL)
    w = workloads.custom(RUN_LENS, 16, dtype=dtype, window=window | vlf.CAUSAL, base=1.6e5,
                         table_rows=9000, seed=43)
    qkv, cos, sin = inputs(w)
    _say(f"case causal window runs {dtype} W={window}")
    out, lse = run_gpu(w, qkv, cos, sin, br=256, prerotate=False)
    rows = sample_rows(w, 256, 1500, seed=5)
    compare(f"causal ring {dtype} W={window} ({len(rows)} rows)", w, out, lse, qkv, cos, sin,
            rows=rows)
