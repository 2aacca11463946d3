"""GPU parity of the backward (vlf_attend_backward through the C ABI) against the oracle's
float64 gradient (mode B: the same rounded score operands). The forward that feeds it (out, lse)
is the library's own, as in a training step.

The measure is the page's: the largest absolute error over dqkv divided by the largest
magnitude of the oracle's dqkv. The page's backward test bounds it by 3e-2 for bf16 inputs; the
kernel rounds P and dS to the storage type where they enter the matrix products (relative
2^-9 for bf16, 2^-12 for fp16), so fp16 is held to 1e-2."""
import sys

import numpy as np
import pytest
import torch

import oracle
import variable_length_flash_amd as vlf
from variable_length_flash_amd import workloads

pytestmark = pytest.mark.gpu

REL_TOL = {"bf16": 3e-2, "fp16": 1e-2}
GUARD = 4096


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dout(w, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((w.tokens, w.heads * 64)).astype(np.float32)
    return torch.from_numpy(oracle.round_to(x, w.dtype).astype(np.float32)).to(
        torch.bfloat16 if w.dtype == "bf16" else torch.float16)


def run_backward(w, window=None, seed=0, br=64):
    """Forward then backward on cuda:0 on br-row tiles, dqkv in a NaN-filled buffer with a guard
    region."""
    window = w.window if window is None else window
    qkv = workloads.draw_qkv(w)
    cos, sin = workloads.rope_tables(w)
    dout = _dout(w, seed)
    dev = torch.device("cuda:0")
    q, c, s, do = qkv.to(dev), cos.to(dev), sin.to(dev), dout.to(dev)
    out, lse = vlf.attend(q, c, s, w.cu, w.heads, window, w.scale)
    batch = vlf.prepare(w.cu, dev, br, False, window)
    T, H = w.tokens, w.heads
    buf = torch.full((T * 3 * H * 64 + GUARD,), float("nan"), dtype=q.dtype, device=dev)
    dqkv = buf[:T * 3 * H * 64].view(T, 3 * H * 64)
    vlf.attend_backward_into(batch, q, c, s, H, window, w.scale, out, lse, do, dqkv)
    torch.cuda.synchronize()
    assert torch.isnan(buf[T * 3 * H * 64:]).all(), "guard region written"
    return qkv, cos, sin, dout, dqkv.float().cpu().numpy()


def compare(name, w, qkv, cos, sin, dout, got, window=None):
    window = w.window if window is None else window
    want = oracle.attend_backward(qkv.float().numpy(), cos.float().numpy(), sin.float().numpy(),
                                  w.cu, w.heads, window, w.scale, dout.float().numpy(),
                                  mode="B", dtype=w.dtype)
    assert np.isfinite(got).all(), "unwritten or non-finite dqkv"
    top = float(np.abs(want).max())
    err = float(np.abs(got - want).max())
    hd = w.heads * 64
    parts = {k: float(np.abs(got[:, sl] - want[:, sl]).max()) / top
             for k, sl in (("dq", slice(0, hd)), ("dk", slice(hd, 2 * hd)),
                           ("dv", slice(2 * hd, 3 * hd)))}
    _say(f"[backward] {name}: rel {err / top:.2e} (tol {REL_TOL[w.dtype]:.0e}); "
         + ", ".join(f"{k} {v:.2e}" for k, v in parts.items()))
    assert err <= REL_TOL[w.dtype] * top, (name, err / top)


LENS = [5, 40, 1, 33, 70]


@pytest.mark.parametrize("br", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", [0, 9, 65])
def test_backward_page_fixture(dtype, window, br):
    w = workloads.custom(LENS, 2, dtype=dtype, window=window, table_rows=128, seed=7)
    _say(f"case backward page fixture {dtype} W={window} br={br}")
    qkv, cos, sin, dout, got = run_backward(w, seed=1, br=br)
    compare(f"lens {LENS} {dtype} W={window} br={br}", w, qkv, cos, sin, dout, got)


RAGGED = [1, 63, 64, 65, 127, 128, 129, 300, 0, 257, 31, 32, 33, 2]


@pytest.mark.parametrize("br", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 1, 33, 128])
def test_backward_ragged(window, br):
    w = workloads.custom(RAGGED, 3, dtype="bf16", window=window, base=1e4, table_rows=512,
                         seed=11)
    _say(f"case backward ragged W={window} br={br}")
    qkv, cos, sin, dout, got = run_backward(w, seed=2, br=br)
    compare(f"ragged W={window} br={br}", w, qkv, cos, sin, dout, got)


@pytest.mark.parametrize("dtype,window,br", [("bf16", 0, 64), ("fp16", 0, 64),
                                             ("bf16", 300, 64), ("bf16", 0, 128),
                                             ("bf16", 300, 128), ("fp16", 0, 128),
                                             ("bf16", 0, 256), ("bf16", 300, 256),
                                             ("fp16", 0, 256)])
def test_backward_longer_sequences(dtype, window, br):
    """Many steps per tile: each key tile's dK, dV and each query tile's dQ summed over up to
    41 staged steps, through both LDS buffers many times."""
    w = workloads.custom([700, 1300, 64], 2, dtype=dtype, window=window, base=1.6e5,
                         table_rows=1300, seed=19)
    _say(f"case backward longer {dtype} W={window} br={br}")
    qkv, cos, sin, dout, got = run_backward(w, seed=3, br=br)
    compare(f"[700, 1300, 64] {dtype} W={window} br={br}", w, qkv, cos, sin, dout, got)


def test_backward_is_deterministic():
    """Every element of dqkv is written once from sums in registers: two runs agree bit for
    bit."""
    w = workloads.custom([700, 1300, 64], 2, dtype="bf16", window=0, base=1.6e5,
                         table_rows=1300, seed=19)
    _say("case backward determinism")
    a = run_backward(w, seed=3, br=256)[4]
    b = run_backward(w, seed=3, br=256)[4]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("br", [64, 128, 256])
def test_backward_single_key_rows(br):
    """W = 1: each row sees only itself, so dv = dout and dq, dk are zero up to the rounding of
    dP - delta (one key's dO.v against the same product summed by the delta kernel)."""
    w = workloads.custom([1, 7, 130, 64, 300], 2, dtype="bf16", window=1, table_rows=512, seed=5)
    _say(f"case backward single-key rows br={br}")
    qkv, cos, sin, dout, got = run_backward(w, seed=4, br=br)
    hd = w.heads * 64
    d = dout.float().numpy()
    assert np.abs(got[:, 2 * hd:] - d).max() <= 2 ** -8 * np.abs(d).max()
    assert np.abs(got[:, :2 * hd]).max() <= 1e-2


@pytest.mark.parametrize("br", [64, 128])
def test_backward_offsets_past_2gib(br):
    """qkv of 2.2 GB (88 sequences of 1024 tokens, 64 heads, bf16): byte offsets into qkv, dout
    and dqkv pass 2^31. At 128 rows the prep pass's block offsets pass 2^32 and both passes
    build their per-step buffer descriptors from 64-bit row offsets; at 64 rows the passes
    stage every step from qkv and dout themselves, from their own 64-bit row offsets. Inputs drawn on the GPU from a seeded
    generator; the first and the last two sequences (all rows, every head) against the
    oracle."""
    lens, H = [1024] * 88, 64
    w = workloads.custom(lens, H, dtype="bf16", window=0, base=1.6e5, table_rows=1024, seed=23)
    T = w.tokens
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(23)
    q = torch.randn((T, 3 * H * 64), generator=gen, device=dev).to(torch.bfloat16)
    do = torch.randn((T, H * 64), generator=gen, device=dev).to(torch.bfloat16)
    assert q.numel() * 2 > 2 ** 31
    cos, sin = workloads.rope_tables(w)
    c, s = cos.to(dev), sin.to(dev)
    out, lse = vlf.attend(q, c, s, w.cu, H, 0, w.scale)
    _say(f"case backward offsets past 2 GiB br={br}")
    batch = vlf.prepare(w.cu, dev, br, False, 0)
    ws_bytes = vlf.backward_workspace_bytes(T, len(lens), H, br)
    assert ws_bytes > 2 ** 31 or br == 64
    dqkv = torch.full_like(q, float("nan"))
    vlf.attend_backward_into(batch, q, c, s, H, 0, w.scale, out, lse, do, dqkv)
    torch.cuda.synchronize()
    assert not torch.isnan(dqkv).any()
    cu1 = np.array([0, 1024], dtype=np.int32)
    for si in (0, 86, 87):
        a, b = 1024 * si, 1024 * (si + 1)
        want = oracle.attend_backward(q[a:b].float().cpu().numpy(), cos.float().numpy(),
                                      sin.float().numpy(), cu1, H, 0, w.scale,
                                      do[a:b].float().cpu().numpy(), mode="B", dtype="bf16")
        got = dqkv[a:b].float().cpu().numpy()
        rel = float(np.abs(got - want).max() / np.abs(want).max())
        _say(f"[backward] 2.2 GB qkv br={br}, sequence {si}: rel {rel:.2e}")
        assert rel <= REL_TOL["bf16"], (si, rel)


@pytest.mark.parametrize("br", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 1, 33, 200])
def test_backward_causal_window(window, br):
    """The causal mask (keys i - W < j <= i): the key pass sees only queries at or after its
    keys, the query pass only keys at or before its rows."""
    w = workloads.custom(RAGGED + [700], 2, dtype="bf16", window=window | vlf.CAUSAL,
                         base=1.6e5, table_rows=700, seed=13)
    _say(f"case backward causal W={window} br={br}")
    qkv, cos, sin, dout, got = run_backward(w, seed=5, br=br)
    compare(f"causal W={window} br={br}", w, qkv, cos, sin, dout, got)
