"""Pins of the oracle's gradient (``oracle.attend_backward``) to things other than itself:
central differences of the forward oracle, a closed form, a library routine's autograd and an
invariant. CPU only."""
import numpy as np
import pytest

import oracle

LENS = [3, 5, 1]


def _inputs(lens, heads, seed, table_rows=None, unit=False):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    P = table_rows or max(lens)
    qkv = rng.standard_normal((T, 3 * heads * 64)).astype(np.float32)
    if unit:
        cos = np.ones((P, 32), dtype=np.float32)
        sin = np.zeros((P, 32), dtype=np.float32)
    else:
        # any tables, not only rotations: the gradient takes the transpose of whatever linear
        # map the tables define
        cos = rng.uniform(-1.5, 1.5, (P, 32)).astype(np.float32)
        sin = rng.uniform(-1.5, 1.5, (P, 32)).astype(np.float32)
    dout = rng.standard_normal((T, heads * 64))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return qkv, cos, sin, dout, cu


def _loss(qkv, cos, sin, cu, heads, window, scale, dout):
    out, _ = oracle.attend(qkv, cos, sin, cu, heads, window, scale, mode="A")
    return float((out * dout).sum())


@pytest.mark.parametrize("window", [0, 2])
def test_gradient_matches_central_differences(window):
    """Every element of dqkv against (L(x + h) - L(x - h)) / (2h) of the forward oracle (mode A,
    float64), with the step taken on the float32 inputs the oracle reads."""
    heads, scale = 1, 0.3
    qkv, cos, sin, dout, cu = _inputs(LENS, heads, seed=3)
    g = oracle.attend_backward(qkv, cos, sin, cu, heads, window, scale, dout, mode="A")
    flat = qkv.reshape(-1)
    fd = np.zeros(flat.size)
    for k in range(flat.size):
        x0 = flat[k]
        up, dn = np.float32(x0 + 2.0 ** -10), np.float32(x0 - 2.0 ** -10)
        flat[k] = up
        lp = _loss(qkv, cos, sin, cu, heads, window, scale, dout)
        flat[k] = dn
        lm = _loss(qkv, cos, sin, cu, heads, window, scale, dout)
        flat[k] = x0
        fd[k] = (lp - lm) / (float(up) - float(dn))
    err = np.abs(fd - g.reshape(-1)).max()
    assert err <= 2e-5 * max(1.0, np.abs(g).max()), err


def test_single_key_rows():
    """W = 1: every row sees only itself, out = v, so dv = dout exactly and dq = dk = 0."""
    heads = 2
    qkv, cos, sin, dout, cu = _inputs([4, 1, 7], heads, seed=5)
    for mode in ("A", "B"):
        g = oracle.attend_backward(qkv, cos, sin, cu, heads, 1, 0.125, dout, mode=mode)
        hd = heads * 64
        assert np.array_equal(g[:, 2 * hd:], dout)
        assert np.abs(g[:, :2 * hd]).max() == 0.0


@pytest.mark.parametrize("window", [0, 3])
def test_identity_rotation_matches_torch_autograd(window):
    """cos = 1, sin = 0: plain attention per sequence. Against torch autograd (float64, CPU) of
    softmax(scale Q K^T + mask) V."""
    torch = pytest.importorskip("torch")
    heads, scale = 2, 0.2
    lens = [6, 1, 9]
    qkv, cos, sin, dout, cu = _inputs(lens, heads, seed=7, unit=True)
    g = oracle.attend_backward(qkv, cos, sin, cu, heads, window, scale, dout, mode="A")
    hd = heads * 64
    x = torch.tensor(qkv.astype(np.float64), requires_grad=True)
    d = torch.tensor(dout)
    loss = 0.0
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        pos = torch.arange(b - a)
        gap = (pos[:, None] - pos[None, :]).abs()
        mask = torch.zeros(b - a, b - a, dtype=torch.float64)
        if window > 0:
            mask[gap >= window] = float("-inf")
        for h in range(heads):
            q = x[a:b, h * 64:(h + 1) * 64]
            k = x[a:b, hd + h * 64:hd + (h + 1) * 64]
            v = x[a:b, 2 * hd + h * 64:2 * hd + (h + 1) * 64]
            p = torch.softmax(scale * (q @ k.T) + mask, dim=1)
            loss = loss + ((p @ v) * d[a:b, h * 64:(h + 1) * 64]).sum()
    loss.backward()
    assert np.abs(x.grad.numpy() - g).max() <= 1e-12 * max(1.0, np.abs(g).max())


def test_value_gradient_sums_to_the_output_gradient():
    """Each row's probabilities sum to 1, so per (sequence, head) the value gradients sum to the
    sum of dout over the sequence's rows."""
    heads = 3
    qkv, cos, sin, dout, cu = _inputs([10, 2, 17], heads, seed=11)
    hd = heads * 64
    for window in (0, 4):
        g = oracle.attend_backward(qkv, cos, sin, cu, heads, window, 0.125, dout, mode="B")
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            assert np.allclose(g[a:b, 2 * hd:].sum(axis=0), dout[a:b].sum(axis=0),
                               rtol=0, atol=1e-12)


def test_modes_differ_only_by_operand_rounding():
    """bf16 operands move the gradient by little; mode B equals mode A on inputs whose rotated
    operands are already bf16 values (cos = 1, sin = 0, scale a power of two)."""
    heads = 1
    qkv, cos, sin, dout, cu = _inputs([12, 5], heads, seed=13, unit=True)
    qkv = oracle.round_to(qkv, "bf16").astype(np.float32)
    ga = oracle.attend_backward(qkv, cos, sin, cu, heads, 0, 0.125, dout, mode="A")
    gb = oracle.attend_backward(qkv, cos, sin, cu, heads, 0, 0.125, dout, mode="B",
                                dtype="bf16")
    assert np.array_equal(ga, gb)
    qkv2, cos2, sin2, dout2, cu2 = _inputs([12, 5], heads, seed=13)
    qkv2 = oracle.round_to(qkv2, "bf16").astype(np.float32)
    ga = oracle.attend_backward(qkv2, cos2, sin2, cu2, heads, 0, 0.125, dout2, mode="A")
    gb = oracle.attend_backward(qkv2, cos2, sin2, cu2, heads, 0, 0.125, dout2, mode="B",
                                dtype="bf16")
    assert 0 < np.abs(ga - gb).max() <= 5e-2 * np.abs(ga).max()
