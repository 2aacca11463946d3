"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/vlf_oracle.c`` to a temporary directory, plants one plausible mistake
(a flipped sign, a swapped operand, a wrong index or bound, a dropped term), builds that copy
and runs a battery of the pins from test_oracle.py against it. Every mutant must fail at least
one pin; the unmodified source must pass them all.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import brute
import oracle
from variable_length_flash_amd import workloads

SOURCE = os.path.join(os.path.dirname(oracle.__file__), "vlf_oracle.c")
LENS = [5, 40, 1, 33, 70]
HEADS = 2
SCALE = 0.125

MUTANTS = {
    "rotation sign": ("y[m] = x1 * cm - x2 * sm;", "y[m] = x1 * cm + x2 * sm;"),
    "cos/sin swapped": ("y[m + HALF] = x1 * sm + x2 * cm;", "y[m + HALF] = x1 * cm + x2 * sm;"),
    "mode B sign": ("float a = fmaf(x[m], c[m], -(x[m + HALF] * s[m]));",
                    "float a = fmaf(x[m], c[m], (x[m + HALF] * s[m]));"),
    "window bound": ("if ((w > 0 && gap >= w) || (causal && j > i)) {",
                     "if ((w > 0 && gap > w) || (causal && j > i)) {"),
    "causal bound": ("if ((w > 0 && gap >= w) || (causal && j > i)) {",
                     "if ((w > 0 && gap >= w) || (causal && j >= i)) {"),
    "key position global": ("cos_t + j * HALF, sin_t + j * HALF,", "cos_t + t * HALF, sin_t + t * HALF,"),
    "query position global": ("cos_t + i * HALF, sin_t + i * HALF, mode,",
                              "cos_t + t * HALF, sin_t + t * HALF, mode,"),
    "values read from keys": ("(start + j) * ld + 2 * hd + (int64_t)h * HD;",
                              "(start + j) * ld + hd + (int64_t)h * HD;"),
    "lse drops the max": ("double lz = m + log(sum);", "double lz = log(sum) + 0.0 * m;"),
    "mode A scale dropped": ("sc[j] = mode == ORACLE_MODE_A ? scale * dot : dot;",
                             "sc[j] = mode == ORACLE_MODE_A ? dot : dot;"),
    "mode B scale dropped": ("a = a * scale;", "a = a * 1.0f;"),
    "key head offset": ("const double *k = krot + (start + j) * hd + (int64_t)h * HD;",
                        "const double *k = krot + (start + j) * hd;"),
    "pair index": ("double x1 = x[m], x2 = x[m + HALF], cm = c[m], sm = s[m];",
                   "double x1 = x[m], x2 = x[m + HALF], cm = c[m ^ 1], sm = s[m ^ 1];"),
    "ties away from zero": ("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))",
                            "if (frac >= 0.5)"),
    "bf16 precision": ("return round_binary(x, 8, -126, 0x1.fep127, 127);",
                       "return round_binary(x, 9, -126, 0x1.fep127, 127);"),
    "key sequence start": ("int64_t t = cu[s] + j;", "int64_t t = j;"),
}


def _build(tmp_path, name, old, new):
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(path), "-o", str(lib), "-lm"], check=True)
    return str(lib)


def _inputs(dtype, seed=7):
    # tables cover every token index, so mutants that index them by token (not position) read
    # wrong rows, never past the table
    w = workloads.custom(LENS, HEADS, dtype=dtype, table_rows=sum(LENS), seed=seed)
    qkv = workloads.draw_qkv(w).float().numpy()
    cos, sin = workloads.rope_tables(w)
    return w, qkv, cos.float().numpy(), sin.float().numpy()


def _pins_pass(lib) -> bool:
    """True when the library passes every pin of the battery."""
    # rounding against library conversions
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000), 1.0 + (2 * np.arange(-20, 20) + 1) * 2.0 ** -8,
                        1.0 + (2 * np.arange(-20, 20) + 1) * 2.0 ** -11]).astype(np.float32)
    if not np.array_equal(oracle.round_to(x.astype(np.float64), "bf16", library=lib),
                          torch.from_numpy(x).to(torch.bfloat16).double().numpy()):
        return False
    if not np.array_equal(oracle.round_to(x.astype(np.float64), "fp16", library=lib),
                          x.astype(np.float16).astype(np.float64)):
        return False
    # brute force in both modes, both storage types, full and windowed
    for dtype in ("bf16", "fp16"):
        w, qkv, cos, sin = _inputs(dtype)
        for mode in ("A", "B"):
            for window in (0, 9, brute.CAUSAL | 9):
                out, lse = oracle.attend(qkv, cos, sin, w.cu, HEADS, window, SCALE, mode=mode,
                                         dtype=dtype, library=lib)
                bout, blse = brute.attend(qkv, cos, sin, LENS, HEADS, window, SCALE, mode=mode,
                                          dtype=dtype)
                # written so that a NaN anywhere fails the pin
                if not (np.abs(out - bout).max() <= 1e-12 and np.abs(lse - blse).max() <= 1e-12):
                    return False
    return True


def test_unmodified_source_passes(tmp_path):
    lib = _build(tmp_path, "none", "#define HD 64", "#define HD 64")
    assert _pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build(tmp_path, name, old, new)
    assert not _pins_pass(lib), f"planted mistake {name!r} went unnoticed"
