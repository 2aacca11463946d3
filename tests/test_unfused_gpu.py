"""The unfused baseline (vlf_rotate_qkv, then vlf_attend with identity tables and scale 1)
through the C ABI: its rotated operands bit for bit against the oracle's rounded operands
(mode B), and its forward bit for bit against the fused forward on the same schedule."""
import numpy as np
import pytest
import torch

import oracle
import variable_length_flash_amd as vlf
from variable_length_flash_amd import workloads

pytestmark = pytest.mark.gpu

CASES = [([5, 40, 1, 33, 70], 2, "bf16", 9), ([5, 40, 1, 33, 70], 2, "fp16", 0),
         ([1, 63, 64, 65, 127, 128, 129, 300, 0, 257], 3, "bf16", 0),
         ([700, 1300, 64], 2, "fp16", 300)]


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("lens,heads,dtype,window", CASES)
def test_unfused_baseline_rounds_like_the_fused_forward(lens, heads, dtype, window):
    w = workloads.custom(lens, heads, dtype=dtype, window=window, base=1.6e5,
                         table_rows=max(lens), seed=31)
    qkv = workloads.draw_qkv(w)
    cos, sin = workloads.rope_tables(w)
    dev = torch.device("cuda:0")
    q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
    print(f"case unfused {lens} {dtype} W={window}", flush=True)
    hd = heads * 64
    for br in (64, 128, 256):
        batch = vlf.prepare(w.cu, dev, br, False, window)
        dst = torch.zeros_like(q)
        vlf.rotate_qkv_into(batch, q, c, s, heads, w.scale, dst)
        torch.cuda.synchronize()
        qt, kt = oracle.operands(qkv.float().numpy(), cos.float().numpy(), sin.float().numpy(),
                                 w.cu, heads, w.scale, mode="B", dtype=dtype)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        assert np.array_equal(_bits(dst[:, :hd]), _bits(torch.from_numpy(qt).to(tdt)))
        assert np.array_equal(_bits(dst[:, hd:2 * hd]), _bits(torch.from_numpy(kt).to(tdt)))
        assert np.array_equal(_bits(dst[:, 2 * hd:]), _bits(q[:, 2 * hd:]))
    # the forward over the rotated operands with identity tables and scale 1, on each path
    one = torch.ones_like(c)
    zero = torch.zeros_like(s)
    batch = vlf.prepare(w.cu, dev, 64, False, window)
    dst = torch.empty_like(q)
    vlf.rotate_qkv_into(batch, q, c, s, heads, w.scale, dst)
    for br, pre in ((64, False), (128, False), (256, False), (128, True), (256, True)):
        out_f, lse_f = vlf.attend(q, c, s, w.cu, heads, window, w.scale, br=br, prerotate=pre)
        out_u, lse_u = vlf.attend(dst, one, zero, w.cu, heads, window, 1.0, br=br, prerotate=pre)
        torch.cuda.synchronize()
        assert torch.equal(out_f.view(torch.int16), out_u.view(torch.int16)), (br, pre)
        assert torch.equal(lse_f, lse_u), (br, pre)
