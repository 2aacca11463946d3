"""Host logic of the schedule cache (``variable_length_flash_amd.tune``): keys, the pick, and
the JSON round trip. CPU only; the timing itself is in tests/test_tune_gpu.py."""
import numpy as np
import pytest

from variable_length_flash_amd import tune


@pytest.mark.parametrize("n,want", [(0, 1), (1, 1), (2, 2), (3, 4), (64, 64), (65, 128),
                                    (131072, 131072), (18381, 32768)])
def test_pow2(n, want):
    assert tune.pow2(n) == want


def test_shape_key_rounds_tokens_and_longest_up_to_powers_of_two():
    cu = np.array([0, 5, 45, 46, 79, 149], dtype=np.int32)  # the page fixture, T = 149
    key = tune.shape_key(cu, 2, 9, "bf16", "dev")
    assert key == "device=dev,dtype=bf16,heads=2,window=9,tokens=256,longest=128"
    # same buckets, same key; another window, dtype or head count, another key
    assert tune.shape_key(np.array([0, 100, 200]), 2, 9, "bf16", "dev") == \
        "device=dev,dtype=bf16,heads=2,window=9,tokens=256,longest=128"
    assert tune.shape_key(cu, 2, 0, "bf16", "dev") != key
    assert tune.shape_key(cu, 2, 9, "fp16", "dev") != key
    assert tune.shape_key(cu, 4, 9, "bf16", "dev") != key


def test_fastest_takes_the_smallest_time_and_the_first_of_equals():
    assert tune.fastest({"a": 3.0, "b": 1.0, "c": 2.0}) == "b"
    assert tune.fastest({"a": 1.0, "b": 1.0}) == "a"
    with pytest.raises(ValueError):
        tune.fastest({})


def test_candidates():
    names = [tune.forward_name(*c) for c in tune.FORWARD_CANDIDATES]
    assert len(names) == len(set(names)) == 6
    assert tune.BACKWARD_CANDIDATES == (64, 128, 256)


def test_save_and_load_round_trip(tmp_path):
    tune.clear()
    tune._cache[("forward", "k1")] = {"pick": (256, True), "ms": {"br256_workspace": 4.2}}
    tune._cache[("backward", "k1")] = {"pick": 128, "ms": {"br128": 15.0, "br64": 22.0}}
    path = tmp_path / "tuned.json"
    tune.save(str(path))
    tune.clear()
    assert tune.cached("forward", "k1") is None
    assert tune.load(str(path)) == 2
    assert tune.cached("forward", "k1")["pick"] == (256, True)
    assert tune.cached("backward", "k1") == {"pick": 128, "ms": {"br128": 15.0, "br64": 22.0}}
    tune.clear()
