"""Pins for the float64 oracle (CPU only).

Each test ties the oracle to something other than itself: a brute-force dense implementation,
a library routine, a closed form, an invariant of the method, or a hand-derived fixture under
tests/golden/. Definitions follow hanzo-kernel 0.2.42 ``src/packed.rs`` (module contract,
``layout``, ``attend``'s masking and rounding points, and the f64 composite ``attend_ref``).
"""
import math
import os

import numpy as np
import pytest
import torch

import brute
import oracle
import variable_length_flash_amd as vlf
from variable_length_flash_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
LENS = [5, 40, 1, 33, 70]  # the page's test lengths
HEADS = 2
SCALE = 0.125


def _inputs(lens, heads, dtype="bf16", seed=7, base=1e4, table_rows=128):
    w = workloads.custom(lens, heads, dtype=dtype, base=base, table_rows=table_rows, seed=seed)
    qkv = workloads.draw_qkv(w).float().numpy()
    cos, sin = workloads.rope_tables(w)
    return w, qkv, cos.float().numpy(), sin.float().numpy()


# ---------------------------------------------------------------- rounding (library conversions)

def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties: 1 + (2k+1) * 2^-8 sits halfway between bf16 neighbours
        1.0 + (2 * np.arange(-50, 50) + 1) * 2.0 ** -8,
        [0.0, -0.0, 3.0e38, -3.0e38, 1e-40, -1e-42],
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, want)


def test_round_fp16_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        1.0 + (2 * np.arange(-50, 50) + 1) * 2.0 ** -11,
        (2 * np.arange(0, 50) + 1) * 2.0 ** -25,  # subnormal ties
        [0.0, 65504.0, 65519.0, 65520.0, -65520.0, 1e6],
    ]).astype(np.float32)
    want = x.astype(np.float16).astype(np.float64)
    got = oracle.round_to(x.astype(np.float64), "fp16")
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- brute force on tiny inputs

@pytest.mark.parametrize("window", [0, 1, 2, 9, 65])
@pytest.mark.parametrize("mode", ["A", "B"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_matches_brute_force(window, mode, dtype):
    w, qkv, cos, sin = _inputs(LENS, HEADS, dtype=dtype)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, window, SCALE, mode=mode, dtype=dtype)
    bout, blse = brute.attend(qkv, cos, sin, LENS, HEADS, window, SCALE, mode=mode, dtype=dtype)
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 1, 2, 9, 65])
@pytest.mark.parametrize("mode", ["A", "B"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_causal_matches_brute_force(window, mode, dtype):
    """The causal window (j <= i, and i - j < W for W >= 1) against the explicit-mask brute
    force."""
    w, qkv, cos, sin = _inputs(LENS, HEADS, dtype=dtype)
    win = window | oracle.CAUSAL
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, win, SCALE, mode=mode, dtype=dtype)
    bout, blse = brute.attend(qkv, cos, sin, LENS, HEADS, win, SCALE, mode=mode, dtype=dtype)
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_causal_first_rows_see_only_themselves():
    """Row 0 of every sequence has one visible key under the causal mask: out = v_0 exactly and
    lse = its own score (mode A: scale * <rot q, rot k>)."""
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, oracle.CAUSAL, SCALE, mode="A")
    hd = HEADS * 64
    for s, L in enumerate(LENS):
        if L == 0:
            continue
        a = int(w.cu[s])
        np.testing.assert_array_equal(out[a], qkv[a, 2 * hd:].astype(np.float64))
        qt, kt = oracle.operands(qkv[a:a + 1], cos, sin, np.array([0, 1]), HEADS, SCALE,
                                 mode="A")
        for h in range(HEADS):
            own = float(qt[0, h * 64:(h + 1) * 64] @ kt[0, h * 64:(h + 1) * 64])
            assert abs(lse[h, a] - own) <= 1e-12 * max(1.0, abs(own))


def test_row_subset_equals_full():
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, 9, SCALE)
    rows = np.array([148, 0, 45, 46, 5, 79, 78, 3], dtype=np.int64)
    sout, slse = oracle.attend(qkv, cos, sin, w.cu, HEADS, 9, SCALE, rows=rows)
    np.testing.assert_array_equal(sout, out[rows])
    np.testing.assert_array_equal(slse, lse[:, rows])


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("window", [0, 3, 17])
def test_identity_rotation_is_plain_attention(window):
    """cos = 1, sin = 0 makes the rotation the identity: per sequence the result is PyTorch's
    scaled_dot_product_attention with a boolean |i-j| < W mask, and the LSE is torch.logsumexp
    of the masked scaled scores."""
    lens = [7, 30, 1, 12]
    heads = 3
    w, qkv, _, _ = _inputs(lens, heads)
    cos = np.ones((64, 32), np.float32)
    sin = np.zeros((64, 32), np.float32)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, heads, window, SCALE, mode="A")
    x = torch.from_numpy(qkv).double()
    hd = heads * 64
    for s, L in enumerate(lens):
        a = int(w.cu[s])
        q = x[a:a + L, :hd].reshape(L, heads, 64).transpose(0, 1)
        k = x[a:a + L, hd:2 * hd].reshape(L, heads, 64).transpose(0, 1)
        v = x[a:a + L, 2 * hd:].reshape(L, heads, 64).transpose(0, 1)
        pos = torch.arange(L)
        mask = torch.ones(L, L, dtype=torch.bool) if window == 0 else \
            (pos[:, None] - pos[None, :]).abs() < window
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                               scale=SCALE)
        got = torch.from_numpy(out[a:a + L]).reshape(L, heads, 64).transpose(0, 1)
        torch.testing.assert_close(got, ref, rtol=0, atol=1e-12)
        sc = (q @ k.transpose(1, 2)) * SCALE
        sc = sc.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(sc, dim=-1)
        torch.testing.assert_close(torch.from_numpy(lse[:, a:a + L]), ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 3])
def test_identity_rotation_causal_is_plain_attention(window):
    """cos = 1, sin = 0 under the causal mask: PyTorch's scaled_dot_product_attention with
    is_causal=True (W = 0), or with the boolean mask 0 <= i - j < W."""
    lens = [7, 30, 1, 12]
    heads = 2
    w, qkv, _, _ = _inputs(lens, heads)
    cos = np.ones((64, 32), np.float32)
    sin = np.zeros((64, 32), np.float32)
    out, _ = oracle.attend(qkv, cos, sin, w.cu, heads, window | oracle.CAUSAL, SCALE, mode="A")
    x = torch.from_numpy(qkv).double()
    hd = heads * 64
    for s, L in enumerate(lens):
        a = int(w.cu[s])
        q = x[a:a + L, :hd].reshape(L, heads, 64).transpose(0, 1)
        k = x[a:a + L, hd:2 * hd].reshape(L, heads, 64).transpose(0, 1)
        v = x[a:a + L, 2 * hd:].reshape(L, heads, 64).transpose(0, 1)
        if window == 0:
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                                   scale=SCALE)
        else:
            pos = torch.arange(L)
            d = pos[:, None] - pos[None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, attn_mask=(d >= 0) & (d < window), scale=SCALE)
        got = torch.from_numpy(out[a:a + L]).reshape(L, heads, 64).transpose(0, 1)
        torch.testing.assert_close(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("window", [0, 1, 4, 13, 200])
def test_zero_queries_give_uniform_weights(window):
    """q = 0 makes every score 0: lse_i = ln n_i and out_i is the mean of the visible values,
    with n_i = min(L, i + W) - max(0, i - W + 1) (W > 0) or L."""
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    qkv[:, :HEADS * 64] = 0.0
    for mode in ("A", "B"):
        out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, window, SCALE, mode=mode)
        for s, L in enumerate(LENS):
            a = int(w.cu[s])
            for i in range(L):
                lo = 0 if window == 0 else max(0, i - window + 1)
                hi = L if window == 0 else min(L, i + window)
                n = hi - lo
                for h in range(HEADS):
                    assert abs(lse[h, a + i] - math.log(n)) < 1e-12
                    v = qkv[a + lo:a + hi, 2 * HEADS * 64 + h * 64:2 * HEADS * 64 + (h + 1) * 64]
                    np.testing.assert_allclose(out[a + i, h * 64:(h + 1) * 64],
                                               v.astype(np.float64).mean(axis=0), atol=1e-12)


def test_single_key_rows():
    """W = 1 (or a length-1 sequence) leaves one visible key, the row's own: out_i = v_i and
    lse_i = scale * <rot(q_i, i), rot(k_i, i)>. Both vectors turn by the same angles, so per
    pair (m, m+32) the product is (c^2 + s^2)(q_m k_m + q_{m+32} k_{m+32}): no rotation needs
    to be applied to write the expected value."""
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, 1, SCALE, mode="A")
    hd = HEADS * 64
    for s, L in enumerate(LENS):
        a = int(w.cu[s])
        for i in range(L):
            c = cos[i].astype(np.float64)
            sn = sin[i].astype(np.float64)
            for h in range(HEADS):
                q = qkv[a + i, h * 64:(h + 1) * 64].astype(np.float64)
                k = qkv[a + i, hd + h * 64:hd + (h + 1) * 64].astype(np.float64)
                want = SCALE * np.sum((c * c + sn * sn) * (q[:32] * k[:32] + q[32:] * k[32:]))
                assert abs(lse[h, a + i] - want) < 1e-12
                np.testing.assert_array_equal(out[a + i, h * 64:(h + 1) * 64],
                                              qkv[a + i, 2 * hd + h * 64:2 * hd + (h + 1) * 64])


def test_constant_values_pass_through():
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    const = np.linspace(-2, 2, 64).astype(np.float32)
    for h in range(HEADS):
        qkv[:, 2 * HEADS * 64 + h * 64:2 * HEADS * 64 + (h + 1) * 64] = const
    for window in (0, 5):
        out, _ = oracle.attend(qkv, cos, sin, w.cu, HEADS, window, SCALE)
        for h in range(HEADS):
            np.testing.assert_allclose(out[:, h * 64:(h + 1) * 64],
                                       np.broadcast_to(const, (w.tokens, 64)), atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_relative_positions_only():
    """Shifting every position by the same offset leaves the scores unchanged (the rotation is
    relative): tables built from exact f64 trig and offset by 37 rows agree to rounding."""
    lens = [20, 9]
    w, qkv, _, _ = _inputs(lens, HEADS)
    p = np.arange(200, dtype=np.float64)[:, None]
    m = np.arange(32, dtype=np.float64)[None, :]
    ang = p / 10000.0 ** (2 * m / 64)
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    a_out, a_lse = oracle.attend(qkv, cos[:100], sin[:100], w.cu, HEADS, 0, SCALE, mode="A")
    b_out, b_lse = oracle.attend(qkv, cos[37:137], sin[37:137], w.cu, HEADS, 0, SCALE, mode="A")
    np.testing.assert_allclose(a_out, b_out, atol=2e-6)
    np.testing.assert_allclose(a_lse, b_lse, atol=2e-6)


@pytest.mark.parametrize("mode", ["A", "B"])
def test_packed_equals_each_alone(mode):
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, 9, SCALE, mode=mode)
    for s, L in enumerate(LENS):
        a = int(w.cu[s])
        cu1 = np.array([0, L], np.int32)
        o1, l1 = oracle.attend(qkv[a:a + L], cos, sin, cu1, HEADS, 9, SCALE, mode=mode)
        np.testing.assert_array_equal(o1, out[a:a + L])
        np.testing.assert_array_equal(l1, lse[:, a:a + L])


def test_permuting_sequences_permutes_rows():
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, 0, SCALE)
    perm = [3, 0, 4, 2, 1]
    pieces = [np.arange(w.cu[s], w.cu[s + 1]) for s in perm]
    idx = np.concatenate(pieces)
    lens2 = [LENS[s] for s in perm]
    cu2 = np.concatenate([[0], np.cumsum(lens2)]).astype(np.int32)
    o2, l2 = oracle.attend(qkv[idx], cos, sin, cu2, HEADS, 0, SCALE)
    np.testing.assert_array_equal(o2, out[idx])
    np.testing.assert_array_equal(l2, lse[:, idx])


def test_wide_window_is_full_attention():
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    full = oracle.attend(qkv, cos, sin, w.cu, HEADS, 0, SCALE)
    wide = oracle.attend(qkv, cos, sin, w.cu, HEADS, max(LENS), SCALE)
    np.testing.assert_array_equal(full[0], wide[0])
    np.testing.assert_array_equal(full[1], wide[1])
    narrower = oracle.attend(qkv, cos, sin, w.cu, HEADS, max(LENS) - 1, SCALE)
    assert np.abs(narrower[1] - full[1]).max() > 0  # the window does bite one step below


@pytest.mark.parametrize("window", [0, 9])
def test_softmax_rows_sum_to_one(window):
    """sum over visible j of exp(s_ij - lse_i) = 1, with the scores formed explicitly."""
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    _, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, window, SCALE, mode="A")
    sc = brute.scores(qkv, cos, sin, LENS, HEADS, window, SCALE, mode="A")
    for s, L in enumerate(LENS):
        a = int(w.cu[s])
        for h in range(HEADS):
            p = np.exp(sc[s][h] - lse[h, a:a + L][:, None])
            np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)


def test_mode_b_is_close_to_mode_a():
    """Rounding the operands to bf16 moves the scores by a few 1e-3 at most on these inputs."""
    w, qkv, cos, sin = _inputs(LENS, HEADS)
    a = oracle.attend(qkv, cos, sin, w.cu, HEADS, 0, SCALE, mode="A")
    b = oracle.attend(qkv, cos, sin, w.cu, HEADS, 0, SCALE, mode="B")
    assert 0 < np.abs(a[1] - b[1]).max() < 3e-2
    assert np.abs(a[0] - b[0]).max() < 3e-2


def test_rejects_bad_cu():
    w, qkv, cos, sin = _inputs([4, 4], 1)
    with pytest.raises(ValueError):
        oracle.attend(qkv, cos, sin, np.array([0, 5, 8], np.int32)[[0, 2, 1]], 1, 0, SCALE)
    with pytest.raises(ValueError):
        oracle.attend(qkv, cos[:3], sin[:3], w.cu, 1, 0, SCALE)  # table shorter than a sequence


# ---------------------------------------------------------------- tile table and pair count

def _golden_tiles():
    table = {}
    with open(os.path.join(HERE, "golden", "tiles_lens_5_40_1_33_70.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            br, rest = line.split(":")
            pairs = [tuple(int(v) for v in p.split(",")) for p in rest.split()]
            table[int(br)] = np.array(pairs, dtype=np.uint32)
    return table


def test_tile_table_golden():
    cu = np.concatenate([[0], np.cumsum(LENS)])
    for br, want in _golden_tiles().items():
        np.testing.assert_array_equal(oracle.tile_table(cu, br), want)


@pytest.mark.parametrize("seed", range(5))
def test_tile_table_brute(seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 40)))]
    cu = np.concatenate([[0], np.cumsum(lens)])
    for br in (16, 64, 128):
        np.testing.assert_array_equal(oracle.tile_table(cu, br), brute.tile_table(lens, br))


def test_pair_count_golden():
    with open(os.path.join(HERE, "golden", "pairs.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            lens, window, want = [x.strip() for x in line.split(";")]
            lens = [int(x) for x in lens.split(",")]
            cu = np.concatenate([[0], np.cumsum(lens)])
            assert oracle.visible_pairs(cu, int(window)) == int(want)
            assert brute.pair_count(lens, int(window)) == int(want)


@pytest.mark.parametrize("lens,window", [([5, 40, 1, 33, 70], 0), ([5, 40, 1, 33, 70], 9),
                                         ([300, 0, 64, 65], 64), ([1, 2, 3], 1)])
def test_causal_pair_count_brute(lens, window):
    cu = np.concatenate([[0], np.cumsum(lens)])
    win = window | oracle.CAUSAL
    assert oracle.visible_pairs(cu, win) == brute.pair_count(lens, win)
    assert vlf.visible_pairs(cu, win) == brute.pair_count(lens, win)


@pytest.mark.parametrize("L,W", [(8192, 0), (8192, 128), (100, 128), (128, 128), (5000, 1)])
def test_causal_pair_count_closed_form(L, W):
    """Row i sees min(i + 1, W) keys (W = 0: i + 1)."""
    want = L * (L + 1) // 2 if W == 0 or L <= W else W * (W + 1) // 2 + (L - W) * W
    assert oracle.visible_pairs([0, L], W | oracle.CAUSAL) == want


@pytest.mark.parametrize("L,W", [(8192, 128), (600, 128), (128, 128), (5000, 1), (1000, 999)])
def test_pair_count_closed_form(L, W):
    """For L >= W a sequence has L(2W - 1) - W(W - 1) visible pairs."""
    assert oracle.visible_pairs([0, L], W) == L * (2 * W - 1) - W * (W - 1)
    assert oracle.visible_pairs([0, L], 0) == L * L
