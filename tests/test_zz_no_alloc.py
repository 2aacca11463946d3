"""vlf_attend_static, the forward for callers that cannot allocate device memory, against the
entry point it mirrors (vlf_attend with a workspace of its own), through the C ABI.

Both run the same two kernels (key tiles, then the forward over them) on the same inputs, so
their outputs must agree bit for bit; each is also held to the oracle's tolerances (mode B: out
within 2e-2 for bf16 and 4e-3 for fp16, lse within 1e-3). Two calls run in a row on one device,
the second on a smaller batch, so the second reads a fixed array the first left full of its own
key tiles: a block it failed to rewrite would show."""
import sys

import numpy as np
import pytest
import torch

import oracle
import variable_length_flash_amd as vlf
from variable_length_flash_amd import binding, workloads

pytestmark = pytest.mark.gpu

OUT_TOL = {"bf16": 2e-2, "fp16": 4e-3}
LSE_TOL = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _forward(w, q, c, s, br, static):
    dev = q.device
    batch = vlf.prepare(w.cu, dev, br, True, w.window)
    assert batch.prerotate and batch.br == br
    out = torch.full((w.tokens, w.heads * 64), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((w.heads, w.tokens), float("nan"), dtype=torch.float32, device=dev)
    if static:
        binding.attend_static_into(batch, q, c, s, w.heads, w.window, w.scale, out, lse)
    else:
        ws = torch.empty(vlf.workspace_bytes(w.tokens, w.sequences, w.heads), dtype=torch.uint8,
                         device=dev)
        vlf.attend_into(batch, q, c, s, w.heads, w.window, w.scale, out, lse, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


def test_static_workspace_matches_the_allocating_entry_point():
    dev = torch.device("cuda:0")
    big = workloads.custom([3000, 1700, 900, 64, 1], 4, dtype="bf16", window=0, base=1.6e5,
                           table_rows=3000, seed=51)
    small = workloads.custom([700, 300, 65], 2, dtype="fp16", window=300, base=1e4,
                             table_rows=700, seed=52)
    for w, br in ((big, 256), (small, 128)):
        need = vlf.workspace_bytes(w.tokens, w.sequences, w.heads)
        assert need <= binding.STATIC_WORKSPACE_BYTES
        qkv = workloads.draw_qkv(w)
        cos, sin = workloads.rope_tables(w)
        q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
        _say(f"case static workspace T={w.tokens} H={w.heads} {w.dtype} W={w.window} br={br}")
        want_out, want_lse = _forward(w, q, c, s, br, static=False)
        got_out, got_lse = _forward(w, q, c, s, br, static=True)
        assert not torch.isnan(got_out).any() and not torch.isnan(got_lse).any()
        assert torch.equal(got_out, want_out) and torch.equal(got_lse, want_lse)
        o_out, o_lse = oracle.attend(qkv.float().numpy(), cos.float().numpy(),
                                     sin.float().numpy(), w.cu, w.heads, w.window, w.scale,
                                     mode="B", dtype=w.dtype)
        e_out = float(np.abs(got_out.float().cpu().numpy() - o_out).max())
        e_lse = float(np.abs(got_lse.cpu().numpy() - o_lse).max())
        _say(f"[static] T={w.tokens}: bit-identical to vlf_attend with a workspace; oracle out "
             f"{e_out:.2e}, lse {e_lse:.2e}")
        assert e_out <= OUT_TOL[w.dtype] and e_lse <= LSE_TOL


def test_static_workspace_rejects_a_batch_beyond_its_size():
    """The long workload's key tiles need 541 MB, beyond the 128 MiB array: refused with a
    message before anything is launched."""
    dev = torch.device("cuda:0")
    w = workloads.long()
    assert vlf.workspace_bytes(w.tokens, w.sequences, w.heads) > binding.STATIC_WORKSPACE_BYTES
    batch = vlf.prepare(w.cu, dev, 256, True, 0)
    q = torch.empty((w.tokens, 3 * w.heads * 64), dtype=torch.bfloat16, device=dev)
    c = torch.empty((8192, 32), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w.tokens, w.heads * 64), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.heads, w.tokens), dtype=torch.float32, device=dev)
    with pytest.raises(vlf.VlfError) as err:
        binding.attend_static_into(batch, q, c, c, w.heads, 0, w.scale, out, lse)
    assert err.value.status == binding.VLF_EINVAL and "exceeds the static array" in str(err.value)
