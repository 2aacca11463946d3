"""The schedule cache on the GPU: every candidate timed once per shape key, the pick reused, and
the tuned forward and backward against the oracle (mode B), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from variable_length_flash_amd import tune, workloads

pytestmark = pytest.mark.gpu


def _inputs(w):
    qkv = workloads.draw_qkv(w)
    cos, sin = workloads.rope_tables(w)
    return qkv, cos, sin


def test_forward_tuning_times_each_candidate_once_and_matches_the_oracle(monkeypatch):
    tune.clear()
    w = workloads.custom([5, 40, 1, 33, 70, 300], 2, dtype="bf16", window=9, table_rows=300,
                         seed=7)
    qkv, cos, sin = _inputs(w)
    dev = torch.device("cuda:0")
    q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
    print("case forward tuning", flush=True)
    out, lse = tune.attend_tuned(q, c, s, w.cu, w.heads, w.window, w.scale)
    key = tune.shape_key(w.cu, w.heads, w.window, "bf16", torch.cuda.get_device_name(dev))
    entry = tune.cached("forward", key)
    assert entry["pick"] in tune.FORWARD_CANDIDATES
    assert len(entry["ms"]) == 6 and all(v > 0 for v in entry["ms"].values())
    # a second call with the same key times nothing
    monkeypatch.setattr(tune, "_time", lambda *a, **k: (_ for _ in ()).throw(AssertionError))
    out2, lse2 = tune.attend_tuned(q, c, s, w.cu, w.heads, w.window, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    want_out, want_lse = oracle.attend(qkv.float().numpy(), cos.float().numpy(),
                                       sin.float().numpy(), w.cu, w.heads, w.window, w.scale,
                                       mode="B", dtype="bf16")
    assert np.abs(out.float().cpu().numpy() - want_out).max() <= 2e-2
    assert np.abs(lse.cpu().numpy() - want_lse).max() <= 1e-3
    tune.clear()


def test_backward_tuning_matches_the_oracle():
    tune.clear()
    w = workloads.custom([700, 1, 300, 64], 2, dtype="bf16", window=0, base=1.6e5,
                         table_rows=700, seed=19)
    qkv, cos, sin = _inputs(w)
    dev = torch.device("cuda:0")
    q, c, s = qkv.to(dev), cos.to(dev), sin.to(dev)
    rng = np.random.default_rng(3)
    dout = torch.from_numpy(oracle.round_to(rng.standard_normal((w.tokens, w.heads * 64))
                                            .astype(np.float32), "bf16").astype(np.float32))
    do = dout.to(dev, torch.bfloat16)
    print("case backward tuning", flush=True)
    out, lse = tune.attend_tuned(q, c, s, w.cu, w.heads, 0, w.scale)
    dqkv = tune.attend_backward_tuned(q, c, s, w.cu, w.heads, out, lse, do, 0, w.scale)
    torch.cuda.synchronize()
    key = tune.shape_key(w.cu, w.heads, 0, "bf16", torch.cuda.get_device_name(dev))
    assert tune.cached("backward", key)["pick"] in tune.BACKWARD_CANDIDATES
    want = oracle.attend_backward(qkv.float().numpy(), cos.float().numpy(), sin.float().numpy(),
                                  w.cu, w.heads, 0, w.scale, dout.numpy(), mode="B", dtype="bf16")
    got = dqkv.float().cpu().numpy()
    assert np.abs(got - want).max() <= 3e-2 * np.abs(want).max()
    tune.clear()
