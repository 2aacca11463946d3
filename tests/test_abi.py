"""The C-ABI library on the CPU: it loads, exports every function include/vlf.h declares, builds
the tile table and the pair count bit-exactly, and rejects malformed arguments with a status and
a message before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import variable_length_flash_amd as vlf
from variable_length_flash_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="vlf.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vlf_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(binding.EXPORTS)


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["vlf.h", "vlf_probe.h"]


def test_probe_library_exports_its_header():
    from variable_length_flash_amd import probe
    assert _declared("vlf_probe.h") == sorted(probe.EXPORTS)
    lib = probe.load_library()
    for name in probe.EXPORTS:
        assert hasattr(lib, name), name
    # argument errors come back before any launch
    assert lib.vlf_probe_mfma(0, 512, 0x1000, None) == -1
    assert "iters" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_mfma(10, 512, 0x1004, None) == -1
    assert "aligned" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_overlap(11, 0, 10, 256, 0x1000, 0x1000, None) == -1
    assert "roles" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_overlap(1, 1, 0, 256, 0x1000, 0x1000, None) == -1
    assert "iters" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_overlap(1, 1, 10, 256, 0x1002, 0x1000, None) == -1
    assert "aligned" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_schedule(10, 8, 256, 0x1000, 0x1000, None) == -1
    assert "kind" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_schedule(0, 6, 256, 0x1000, 0x1000, None) == -1
    assert "steps" in lib.vlf_probe_last_error().decode()
    assert lib.vlf_probe_schedule(0, 8, 256, 0x1000, 0x1004, None) == -1
    assert "aligned" in lib.vlf_probe_last_error().decode()


def test_library_exports_every_declared_function():
    lib = vlf.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.vlf_version() == 5


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIBRARY", str(tmp_path / "absent.so"))
    with pytest.raises(vlf.VlfError):
        binding.load_library()


def _random_cu(rng, count, lo, hi):
    lens = rng.integers(lo, hi + 1, size=count)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), [int(x) for x in lens]


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("br", [1, 16, 64, 128])
def test_tile_table_bit_exact(seed, br):
    rng = np.random.default_rng(seed)
    cu, _ = _random_cu(rng, int(rng.integers(1, 200)), 0, 700)
    got = vlf.tile_table(cu, br)
    want = oracle.tile_table(cu, br)
    assert got.dtype == np.uint32
    np.testing.assert_array_equal(got, want)
    n, m = vlf.tile_count(cu, br)
    assert n == want.shape[0] and m == int(np.diff(cu).max())


def test_tile_table_golden():
    cu = [0, 5, 45, 46, 79, 149]  # the page's lengths 5, 40, 1, 33, 70
    want = {16: [(0, 0), (1, 0), (1, 16), (1, 32), (2, 0), (3, 0), (3, 16), (3, 32), (4, 0),
                 (4, 16), (4, 32), (4, 48), (4, 64)],
            64: [(0, 0), (1, 0), (2, 0), (3, 0), (4, 0), (4, 64)]}
    for br, pairs in want.items():
        assert vlf.tile_table(cu, br).tolist() == [list(p) for p in pairs]


def test_empty_batches():
    assert vlf.tile_table([0], 64).shape == (0, 2)
    assert vlf.tile_table([0, 0, 0], 128).shape == (0, 2)
    assert vlf.visible_pairs([0], 0) == 0
    assert vlf.tile_table([0, 0, 3, 3], 64).tolist() == [[1, 0]]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("window", [0, 1, 2, 9, 64, 128, 129, 10000])
def test_visible_pairs_exact(seed, window):
    rng = np.random.default_rng(100 + seed)
    cu, _ = _random_cu(rng, int(rng.integers(1, 60)), 0, 900)
    assert vlf.visible_pairs(cu, window) == oracle.visible_pairs(cu, window)


def test_visible_pairs_of_the_named_workloads():
    from variable_length_flash_amd import workloads
    for make in workloads.WORKLOADS.values():
        w = make()
        assert vlf.visible_pairs(w.cu, w.window) == oracle.visible_pairs(w.cu, w.window)
    assert vlf.visible_pairs(workloads.long().cu, 0) == 16 * 8192 * 8192


@pytest.mark.parametrize("cu,S,T,msg", [
    ([1, 5], 1, 5, "cu[0]"),
    ([0, 5, 3], 2, 3, "decreases"),
    ([0, 5, 9], 2, 10, "expected T"),
    ([0, 5], -1, 5, "negative"),
])
def test_bad_cu_is_rejected(cu, S, T, msg):
    lib = vlf.load_library()
    arr = np.array(cu, dtype=np.int32)
    n = ctypes.c_int32()
    rc = lib.vlf_tile_count(arr.ctypes.data_as(ctypes.c_void_p), S, T, 64, ctypes.byref(n), None)
    assert rc == binding.VLF_EINVAL
    assert msg in lib.vlf_last_error().decode()


def test_tile_table_capacity_is_checked():
    lib = vlf.load_library()
    cu = np.array([0, 300], dtype=np.int32)
    buf = np.zeros(4, dtype=np.uint32)  # 3 tiles of 128 need 6 slots
    rc = lib.vlf_tile_table(cu.ctypes.data_as(ctypes.c_void_p), 1, 300, 128,
                            buf.ctypes.data_as(ctypes.c_void_p), 4)
    assert rc == binding.VLF_EINVAL and "capacity" in lib.vlf_last_error().decode()


def _attend_status(**kw):
    """Call vlf_attend with fake (never dereferenced) pointers: every case below must be
    rejected on the host before any launch."""
    args = dict(qkv=0x1000, cos=0x2000, sin=0x3000, P=64, max_len=60, cu=0x4000, tiles=0x5000,
                nt=4, br=64, T=100, S=2, H=2, window=0, scale=0.125, dtype=binding.VLF_BF16,
                ws=None, ws_bytes=0, out=0x6000, lse=0x7000, stream=None)
    args.update(kw)
    lib = vlf.load_library()
    rc = lib.vlf_attend(args["qkv"], args["cos"], args["sin"], args["P"], args["max_len"],
                        args["cu"], args["tiles"], args["nt"], args["br"], args["T"], args["S"],
                        args["H"], args["window"], args["scale"], args["dtype"], args["ws"],
                        args["ws_bytes"], args["out"], args["lse"], args["stream"])
    return rc, lib.vlf_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=7), binding.VLF_EUNSUPPORTED, "dtype"),
    (dict(br=32), binding.VLF_EUNSUPPORTED, "br"),
    (dict(H=0), binding.VLF_EINVAL, "H ="),
    (dict(H=70000), binding.VLF_EINVAL, "H ="),
    (dict(window=-1), binding.VLF_EINVAL, "window"),
    (dict(T=-5), binding.VLF_EINVAL, "negative"),
    (dict(nt=-1), binding.VLF_EINVAL, "negative"),
    (dict(S=0), binding.VLF_EINVAL, "no sequence"),
    (dict(qkv=None), binding.VLF_EINVAL, "null"),
    (dict(lse=None), binding.VLF_EINVAL, "null"),
    (dict(tiles=None), binding.VLF_EINVAL, "null"),
    (dict(P=0), binding.VLF_EINVAL, "rotary"),
    (dict(P=59), binding.VLF_EINVAL, "the longest sequence has 60"),
    (dict(max_len=-1), binding.VLF_EINVAL, "negative"),
    (dict(max_len=101), binding.VLF_EINVAL, "above T"),
    (dict(scale=float("nan")), binding.VLF_EINVAL, "scale"),
    (dict(scale=float("inf")), binding.VLF_EINVAL, "scale"),
    # T=100, S=2, H=2 need 2 * (1 + 2) blocks of 16 KiB plus 6 norm bounds
    (dict(ws=0x8000, ws_bytes=6 * 16388 - 1), binding.VLF_EINVAL, "workspace of"),
    (dict(ws=0x8000, ws_bytes=0), binding.VLF_EINVAL, "workspace of"),
    (dict(ws=None, ws_bytes=4096), binding.VLF_EINVAL, "without a workspace"),
    (dict(ws=0x8000, ws_bytes=-1), binding.VLF_EINVAL, "workspace_bytes"),
    (dict(ws=0x8004, ws_bytes=6 * 16388), binding.VLF_EINVAL, "16-byte aligned"),
])
def test_attend_rejects_bad_arguments(kw, status, msg):
    rc, text = _attend_status(**kw)
    assert rc == status
    assert msg in text


def test_attend_with_no_work_is_a_no_op():
    # no tiles or no tokens: returns OK without touching the (fake) pointers or the device
    assert _attend_status(nt=0)[0] == binding.VLF_OK
    assert _attend_status(T=0, S=0, nt=0, max_len=0, qkv=None, out=None)[0] == binding.VLF_OK
    for br in (64, 128, 256):  # every tile height the forward serves passes validation
        assert _attend_status(nt=0, br=br)[0] == binding.VLF_OK


@pytest.mark.parametrize("T,S,H", [(0, 0, 1), (1, 1, 1), (63, 1, 1), (64, 1, 1), (100, 2, 2),
                                   (131072, 16, 16), (33000, 1024, 16), (5, 5, 65536)])
def test_workspace_bytes(T, S, H):
    # H * (floor(T / 64) + S) blocks of 16 KiB and as many float32 norm bounds; nothing when
    # there is no token
    want = 0 if T == 0 else H * (T // 64 + S) * (16384 + 4)
    assert vlf.workspace_bytes(T, S, H) == want


@pytest.mark.parametrize("lens", [[1], [64], [65], [5, 40, 1, 33, 70], [0, 64, 0, 128, 1],
                                  [63, 1, 63, 1, 200], [8192] * 3])
def test_workspace_blocks_are_disjoint_and_inside(lens):
    """The block of key tile u of sequence s is floor(cu[s] / 64) + s + u: distinct for all
    (s, u) and below floor(T / 64) + S (so inside vlf_workspace_bytes)."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, S = int(cu[-1]), len(lens)
    blocks = [int(cu[s]) // 64 + s + u for s in range(S) for u in range(-(-lens[s] // 64))]
    assert len(set(blocks)) == len(blocks)
    assert all(0 <= b < T // 64 + S for b in blocks)
    assert vlf.workspace_bytes(T, S, 1) >= (max(blocks) + 1) * 16384


@pytest.mark.parametrize("T,S,H,msg", [(-1, 1, 1, "negative"), (1, 1, 70000, "above")])
def test_workspace_bytes_rejects(T, S, H, msg):
    lib = vlf.load_library()
    out = ctypes.c_int64()
    assert lib.vlf_workspace_bytes(T, S, H, ctypes.byref(out)) == binding.VLF_EINVAL
    assert msg in lib.vlf_last_error().decode()


def _rotate_status(**kw):
    args = dict(qkv=0x1000, cos=0x2000, sin=0x3000, P=64, max_len=60, cu=0x4000, T=100, S=2,
                H=2, dtype=binding.VLF_BF16, ws=0x8000, ws_bytes=6 * 16388, stream=None)
    args.update(kw)
    lib = vlf.load_library()
    rc = lib.vlf_rotate_keys(args["qkv"], args["cos"], args["sin"], args["P"], args["max_len"],
                             args["cu"], args["T"], args["S"], args["H"], args["dtype"],
                             args["ws"], args["ws_bytes"], args["stream"])
    return rc, lib.vlf_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=3), binding.VLF_EUNSUPPORTED, "dtype"),
    (dict(H=0), binding.VLF_EINVAL, "H ="),
    (dict(T=-1), binding.VLF_EINVAL, "negative"),
    (dict(S=0), binding.VLF_EINVAL, "no sequence"),
    (dict(ws=None, ws_bytes=0), binding.VLF_EINVAL, "needs a workspace"),
    (dict(ws_bytes=6 * 16388 - 4), binding.VLF_EINVAL, "workspace of"),
    (dict(cu=None), binding.VLF_EINVAL, "null"),
    (dict(P=0), binding.VLF_EINVAL, "rotary"),
    (dict(P=59), binding.VLF_EINVAL, "the longest sequence has 60"),
])
def test_rotate_keys_rejects_bad_arguments(kw, status, msg):
    rc, text = _rotate_status(**kw)
    assert rc == status
    assert msg in text


def test_rotate_keys_with_no_tokens_is_a_no_op():
    assert _rotate_status(T=0, S=0, max_len=0, qkv=None, ws=None, ws_bytes=0)[0] == binding.VLF_OK


def test_attend_static_rejects_a_workspace_beyond_its_array():
    # the long workload's key tiles (541 MB) exceed the 128 MiB array: refused on the host with
    # both sizes in the message, before the array's address is looked up or anything launched
    lib = vlf.load_library()
    T, S, H = 131072, 16, 16
    assert vlf.workspace_bytes(T, S, H) > binding.STATIC_WORKSPACE_BYTES
    rc = lib.vlf_attend_static(0x1000, 0x2000, 0x3000, 8192, 8192, 0x4000, 0x5000, 512, 256, T,
                               S, H, 0, 0.125, binding.VLF_BF16, 0x6000, 0x7000, None)
    msg = lib.vlf_last_error().decode()
    assert rc == binding.VLF_EINVAL and "exceeds the static array" in msg
    assert str(vlf.workspace_bytes(T, S, H)) in msg and str(binding.STATIC_WORKSPACE_BYTES) in msg
    # argument errors of the forward come back the same way
    rc = lib.vlf_attend_static(0x1000, 0x2000, 0x3000, 64, 60, 0x4000, 0x5000, 4, 64, 100, 2, 0,
                               0, 0.125, binding.VLF_BF16, 0x6000, 0x7000, None)
    assert rc == binding.VLF_EINVAL
    # no work: nothing looked up, nothing launched
    assert lib.vlf_attend_static(None, None, None, 0, 0, None, None, 0, 64, 0, 0, 2, 0, 0.125,
                                 binding.VLF_BF16, None, None, None) == binding.VLF_OK


def test_static_workspace_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "vlf.h")).read()
    assert "#define VLF_STATIC_WORKSPACE_BYTES (128LL << 20)" in text
    assert binding.STATIC_WORKSPACE_BYTES == 128 << 20


def test_attend_rotated_needs_a_workspace():
    lib = vlf.load_library()
    rc = lib.vlf_attend_rotated(0x1000, 0x2000, 0x3000, 64, 60, 0x4000, 0x5000, 4, 64, 100, 2,
                                2, 0, 0.125, binding.VLF_BF16, None, 0, 0x6000, 0x7000, None)
    assert rc == binding.VLF_EINVAL and "needs a workspace" in lib.vlf_last_error().decode()


@pytest.mark.parametrize("max_len,window,typical,br", [
    (1, 0, None, 64), (64, 0, None, 64), (65, 0, None, 128), (255, 0, None, 128),
    (513, 0, 447.0, 128), (513, 0, 448.0, 256), (8192, 0, None, 256), (8192, 512, None, 128),
    (8192, 513, None, 256), (64, 128, None, 64),
    # windows of at most 129 keys: 256-row tiles on the key ring once sequences fill them
    (8192, 1, None, 256), (8192, 128, None, 256), (8192, 129, None, 256), (8192, 130, None, 128),
    (8192, 128, 255.0, 128), (300, 128, 256.0, 256),
    # sequences of at most 512 tokens fit the key ring whole: 256-row tiles once typical >= 256
    (256, 0, None, 256), (447, 0, None, 256), (512, 0, 343.0, 256), (512, 600, 300.0, 256),
    # the typical length decides, not the longest sequence
    (600, 0, 343.0, 128), (512, 0, 512.0, 256), (8192, 0, 300.0, 128), (65, 0, 30.0, 128)])
def test_choose_br(max_len, window, typical, br):
    assert vlf.choose_br(max_len, window, typical) == br


@pytest.mark.parametrize("length,br,window,pre", [
    (8192, 256, 0, True), (512, 128, 0, True), (383, 128, 0, False), (343, 128, 0, False),
    (8192, 128, 128, False), (8192, 128, 129, True), (64, 64, 0, False), (448, 256, 0, True),
    (447, 256, 0, False), (2048, 256, 600, True), (8192, 256, 128, False),
    (8192, 256, 129, False), (8192, 256, 130, True)])
def test_choose_prerotate(length, br, window, pre):
    # the workspace pays when a query tile's key span (the typical length, or br + 2W - 1) is
    # three query tiles at 128 rows, or 448 tokens at 256 rows
    assert vlf.choose_prerotate(length, br, window) is pre


def test_window_fits_ring():
    # brute force: the key tiles a 256-row tile at i0 (a multiple of 256, far from either
    # sequence end) reaches under window W, against the eight-slot ring
    for window in range(0, 400):
        i0 = 4096
        if window == 0:
            want = False
        else:
            lo = (i0 + 1 - window) // 64 * 64
            hi = i0 + 256 + window - 1
            want = -(-(hi - lo) // 64) <= 8
        assert binding.window_fits_ring(window) is want, window
    assert binding.window_fits_ring(129) and not binding.window_fits_ring(130)


def test_launch_table_interleaves_whole_sequences_by_cost():
    # by hand, full window, 256-row tiles, every sequence within eight key tiles: an entry costs
    # 2 + the key tiles its rows reach (here the whole sequence). Sequence costs: 0 (512 rows,
    # two entries of 2 + 8) 20, 1 (64) 3, 2 (300, two entries of 2 + 5) 14, 3 (100) 4, 4 (0)
    # none. Most, least, second most, second least: 0, 1, 2, 3.
    lens = [512, 64, 300, 100, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    got = vlf.launch_table(cu, 256, False, 0)
    want = np.array([[0, 0], [0, 256], [1, 0], [2, 0], [2, 256], [3, 0]], dtype=np.uint32)
    np.testing.assert_array_equal(got, want)
    # the other schedules keep the page's order
    for br, pre, window in ((256, True, 0), (128, False, 0), (64, False, 0)):
        np.testing.assert_array_equal(vlf.launch_table(cu, br, pre, window),
                                      vlf.tile_table(cu, br))


@pytest.mark.parametrize("window", [0, 1, 100, 129, 130, 300, 0 | vlf.CAUSAL])
@pytest.mark.parametrize("seed", [0, 1])
def test_launch_table_is_a_permutation_with_sequences_whole(window, seed):
    rng = np.random.default_rng(seed)
    lens = list(rng.integers(0, 513, 60)) + ([3000, 9000] if seed else [])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    canon = vlf.tile_table(cu, 256)
    got = vlf.launch_table(cu, 256, False, window)
    assert got.shape == canon.shape
    # the same entries
    key = lambda t: t[:, 0].astype(np.int64) * 2 ** 32 + t[:, 1]
    np.testing.assert_array_equal(np.sort(key(got)), np.sort(key(canon)))
    # each sequence's entries adjacent and in row order
    seqs = got[:, 0]
    starts = np.nonzero(np.r_[True, seqs[1:] != seqs[:-1]])[0]
    assert len(set(seqs[starts].tolist())) == len(starts)
    for a, b in zip(starts, list(starts[1:]) + [len(got)]):
        np.testing.assert_array_equal(got[a:b, 1], np.arange(b - a) * 256)
    ring = vlf.forward_kernel(256, False, window, max(lens)) == "attend_slide"
    if not ring:
        np.testing.assert_array_equal(got, canon)


def test_launch_table_rejects_what_the_tile_table_rejects():
    lib = vlf.load_library()
    cu = np.array([0, 5, 3], dtype=np.int32)
    buf = np.zeros(16, dtype=np.uint32)
    rc = lib.vlf_launch_table(cu.ctypes.data, 2, 3, 256, 0, 0, buf.ctypes.data, 16)
    assert rc == binding.VLF_EINVAL
    cu = np.array([0, 5], dtype=np.int32)
    assert lib.vlf_launch_table(cu.ctypes.data, 1, 5, 256, 0, -1, buf.ctypes.data, 16) == \
        binding.VLF_EINVAL
    assert "window" in lib.vlf_last_error().decode()
    assert lib.vlf_launch_table(cu.ctypes.data, 1, 5, 256, 0, 0, buf.ctypes.data, 1) == \
        binding.VLF_EINVAL


@pytest.mark.parametrize("lens,want", [([], 0.0), ([0, 0], 0.0), ([5], 5.0), ([100, 156],
                                       (100 ** 2 + 156 ** 2) / 256), ([512] * 32, 512.0)])
def test_typical_length(lens, want):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert vlf.typical_length(cu) == pytest.approx(want)


@pytest.mark.parametrize("name", ["tiny", "encoder", "sliding", "many_short", "long"])
def test_choose_schedule_of_the_workloads(name):
    """The library's whole-batch choice equals its rule on the batch's statistics, and sizes
    the workspace it asks for; the five workloads get the schedules measured best for them."""
    from variable_length_flash_amd import workloads
    w = workloads.WORKLOADS[name]()
    br, pre, max_len, ws = vlf.choose_schedule(w.cu, w.heads, w.window)
    assert max_len == max(w.lens)
    assert (br, pre) == vlf.schedule_rule(max_len, vlf.typical_length(w.cu), w.window)[:2]
    assert ws == (vlf.workspace_bytes(w.tokens, w.sequences, w.heads) if pre else 0)
    want = {"tiny": (128, False), "encoder": (256, False), "sliding": (256, False),
            "many_short": (64, False), "long": (256, True)}[name]
    assert (br, pre) == want
    bbr, bws = vlf.choose_backward(w.cu, w.heads, w.window)
    assert bbr == vlf.choose_backward_br(vlf.typical_length(w.cu))
    assert bws == vlf.backward_workspace_bytes(w.tokens, w.sequences, w.heads, bbr)


@pytest.mark.parametrize("br,pre,window,name", [
    (256, True, 0, "attend_pre_ph"), (128, True, 0, "attend_pre"), (64, True, 128, "attend_pre"),
    (256, False, 128, "attend_slide"), (256, False, 129, "attend_slide"),
    (256, False, 130, "attend_fwd"), (256, False, 0, "attend_fwd"),
    (256, False, 257 | vlf.CAUSAL, "attend_slide"), (256, False, 258 | vlf.CAUSAL, "attend_fwd"),
    (128, False, 128, "attend_fwd"), (64, False, 0, "attend_one"), (32, False, 0, ""),
    (128, False, -1, "")])
def test_forward_kernel_names(br, pre, window, name):
    assert vlf.forward_kernel(br, pre, window) == name


@pytest.mark.parametrize("br,pre,window,max_len,name", [
    (256, False, 0, 512, "attend_slide"), (256, False, 0, 513, "attend_fwd"),
    (256, False, 0 | vlf.CAUSAL, 512, "attend_slide"), (256, False, 600, 300, "attend_slide"),
    (256, False, 600, 1000, "attend_fwd"), (256, False, 100, 100000, "attend_slide"),
    (256, True, 0, 512, "attend_pre_ph"), (128, False, 0, 512, "attend_fwd"),
    (64, False, 0, 64, "attend_one"), (256, False, 0, -1, "")])
def test_forward_kernel_names_by_longest_sequence(br, pre, window, max_len, name):
    # a batch whose sequences all fit eight key tiles keeps each one's whole key range in the
    # ring of attend_slide, whatever the window
    assert vlf.forward_kernel(br, pre, window, max_len) == name


@pytest.mark.parametrize("max_len,typical,window,want", [
    (512, 256.0, 0, (256, 0)), (512, 255.9, 0, (128, 0)), (513, 400.0, 0, (128, 1)),
    (512, 300.0, 300, (256, 0)), (1000, 300.0, 300, (128, 0)), (512, 512.0, 0 | vlf.CAUSAL, (256, 0))])
def test_rule_takes_the_ring_for_sequences_of_at_most_eight_tiles(max_len, typical, window, want):
    br, pre, _ = vlf.schedule_rule(max_len, typical, window)
    assert (br, int(pre)) == want


def test_schedule_calls_reject_bad_arguments():
    lib = vlf.load_library()
    b, p, m = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    ws = ctypes.c_int64()
    bad = np.array([0, 5, 3], dtype=np.int32).ctypes.data_as(ctypes.c_void_p)
    good_arr = np.array([0, 5, 9], dtype=np.int32)
    good = good_arr.ctypes.data_as(ctypes.c_void_p)
    cases = [
        (lambda: lib.vlf_schedule_rule(-1, 10.0, 0, 0, ctypes.byref(b), ctypes.byref(p), None),
         "max_len"),
        (lambda: lib.vlf_schedule_rule(10, -1.0, 0, 0, ctypes.byref(b), ctypes.byref(p), None),
         "typical"),
        (lambda: lib.vlf_schedule_rule(10, 10.0, -1, 0, ctypes.byref(b), ctypes.byref(p), None),
         "window"),
        (lambda: lib.vlf_schedule_rule(10, 10.0, 0, 96, ctypes.byref(b), ctypes.byref(p), None),
         "96"),
        (lambda: lib.vlf_schedule_rule(10, 10.0, 0, 0, None, ctypes.byref(p), None), "null"),
        (lambda: lib.vlf_choose_schedule(bad, 2, 3, 2, 0, ctypes.byref(b), ctypes.byref(p),
                                         ctypes.byref(m), ctypes.byref(ws)), "decreases"),
        (lambda: lib.vlf_choose_schedule(good, 2, 9, 0, 0, ctypes.byref(b), ctypes.byref(p),
                                         None, None), "H ="),
        (lambda: lib.vlf_choose_backward(good, 2, 9, 2, -3, ctypes.byref(b), None), "window"),
        (lambda: lib.vlf_typical_length(good, 2, 9, None), "typical"),
    ]
    for call, text in cases:
        rc = call()
        assert rc == binding.VLF_EINVAL and text in lib.vlf_last_error().decode(), text


def test_tile_count_and_table_at_int32_extremes():
    # one sequence of INT32_MAX - 1 tokens: tile counts for tile heights near INT32_MAX, where
    # the row arithmetic must not wrap in 32 bits
    big = 2 ** 31 - 2
    cu = np.array([0, big], dtype=np.int32)
    for br, want in ((2 ** 31 - 1, 1), (2 ** 30, 2), (big, 1), (big - 1, 2)):
        assert vlf.tile_count(cu, br)[0] == want, br
        table = vlf.tile_table(cu, br)
        assert table.shape == (want, 2)
        assert table[:, 1].tolist() == [i * br for i in range(want)]


@pytest.mark.parametrize("br", [64, 128, 256])
@pytest.mark.parametrize("T,S,H", [(1000, 3, 12), (131072, 16, 16), (1, 1, 1), (63, 63, 2)])
def test_backward_workspace_bytes(T, S, H, br):
    # two float32 [H, T] arrays padded to 256 bytes; above 64 rows, then H * (floor(T / 64) + S)
    # blocks of five 8 KiB images
    floats = (8 * T * H + 255) // 256 * 256
    blocks = 0 if br == 64 else H * (T // 64 + S) * 5 * 8192
    assert vlf.backward_workspace_bytes(T, S, H, br) == floats + blocks


def test_backward_workspace_bytes_rejects():
    assert vlf.backward_workspace_bytes(0, 0, 4, 128) == 0
    lib = vlf.load_library()
    n = ctypes.c_int64(0)
    assert lib.vlf_backward_workspace_bytes(-1, 1, 2, 64, ctypes.byref(n)) == binding.VLF_EINVAL
    assert lib.vlf_backward_workspace_bytes(5, -1, 2, 64, ctypes.byref(n)) == binding.VLF_EINVAL
    assert lib.vlf_backward_workspace_bytes(5, 1, 70000, 64,
                                            ctypes.byref(n)) == binding.VLF_EINVAL
    assert lib.vlf_backward_workspace_bytes(5, 1, 2, 64, None) == binding.VLF_EINVAL
    assert lib.vlf_backward_workspace_bytes(5, 1, 2, 32, ctypes.byref(n)) == binding.VLF_EINVAL


def _backward_status(**kw):
    lib = vlf.load_library()
    cu = np.array([0, 100, 256], dtype=np.int32)
    a = dict(qkv=0x1000, cos=0x2000, sin=0x3000, P=256, max_len=156, cu=cu.ctypes.data,
             tiles=0x4000, num_tiles=5, br=64, T=256, S=2, H=2, W=0, scale=0.125,
             dtype=binding.VLF_BF16, out=0x5000, dout=0x6000, lse=0x7000, ws=0x8000,
             ws_bytes=8 * 256 * 2 + 2 * (256 // 64 + 2) * 5 * 8192, dqkv=0x9000)
    a.update(kw)
    rc = lib.vlf_attend_backward(a["qkv"], a["cos"], a["sin"], a["P"], a["max_len"], a["cu"],
                                 a["tiles"],
                                 a["num_tiles"], a["br"], a["T"], a["S"], a["H"], a["W"],
                                 a["scale"],
                                 a["dtype"], a["out"], a["dout"], a["lse"], a["ws"],
                                 a["ws_bytes"], a["dqkv"], None)
    return rc, lib.vlf_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(dtype=7), binding.VLF_EUNSUPPORTED, "dtype"),
    (dict(W=-1), binding.VLF_EINVAL, "window"),
    (dict(br=512), binding.VLF_EINVAL, "br = 512"),
    (dict(br=32), binding.VLF_EINVAL, "br = 32"),
    (dict(H=0), binding.VLF_EINVAL, "H = 0"),
    (dict(ws_bytes=100), binding.VLF_EINVAL, "workspace"),
    # 64-row tiles need the two float arrays only; taller ones the images as well
    (dict(ws_bytes=8 * 256 * 2 - 1), binding.VLF_EINVAL, "workspace"),
    (dict(br=128, ws_bytes=8 * 256 * 2), binding.VLF_EINVAL, "workspace"),
    (dict(ws=None), binding.VLF_EINVAL, "workspace"),
    (dict(P=155), binding.VLF_EINVAL, "the longest sequence has 156"),
    (dict(ws=0x8008), binding.VLF_EINVAL, "16-byte aligned"),
    (dict(dout=None), binding.VLF_EINVAL, "null device pointer"),
    (dict(dqkv=None), binding.VLF_EINVAL, "null device pointer"),
    (dict(scale=float("nan")), binding.VLF_EINVAL, "scale"),
])
def test_backward_rejects_bad_arguments_before_launching(kw, status, text):
    rc, msg = _backward_status(**kw)
    assert rc == status and text in msg, (rc, msg)


def test_choose_backward_br():
    assert binding.choose_backward_br(0.0) == 64
    assert binding.choose_backward_br(127.9) == 64
    assert binding.choose_backward_br(128.0) == 128
    assert binding.choose_backward_br(8192.0) == 128


def test_backward_with_no_tiles_is_a_no_op():
    assert _backward_status(num_tiles=0, ws=None, ws_bytes=0)[0] == binding.VLF_OK


def test_backward_at_64_rows_takes_the_float_arrays_only():
    # validation passes with exactly the two float arrays; num_tiles = 0 stops before a launch
    assert _backward_status(ws_bytes=8 * 256 * 2, num_tiles=0)[0] == binding.VLF_OK
    lib = vlf.load_library()
    n = ctypes.c_int64(0)
    assert lib.vlf_backward_workspace_bytes(256, 2, 2, 64, ctypes.byref(n)) == binding.VLF_OK
    assert n.value == 8 * 256 * 2


def _rotate_qkv_status(**kw):
    lib = vlf.load_library()
    cu = np.array([0, 100, 256], dtype=np.int32)
    a = dict(qkv=0x1000, cos=0x2000, sin=0x3000, P=256, max_len=156, cu=cu.ctypes.data,
             tiles=0x4000, num_tiles=5, br=64, T=256, S=2, H=2, scale=0.125,
             dtype=binding.VLF_BF16, dst=0x9000)
    a.update(kw)
    rc = lib.vlf_rotate_qkv(a["qkv"], a["cos"], a["sin"], a["P"], a["max_len"], a["cu"],
                            a["tiles"],
                            a["num_tiles"], a["br"], a["T"], a["S"], a["H"], a["scale"],
                            a["dtype"], a["dst"], None)
    return rc, lib.vlf_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(dtype=7), binding.VLF_EUNSUPPORTED, "dtype"),
    (dict(br=32), binding.VLF_EINVAL, "br = 32"),
    (dict(H=0), binding.VLF_EINVAL, "H = 0"),
    (dict(num_tiles=-1), binding.VLF_EINVAL, "negative"),
    (dict(dst=None), binding.VLF_EINVAL, "null device pointer"),
    (dict(tiles=None), binding.VLF_EINVAL, "null device pointer"),
    (dict(dst=0x1000), binding.VLF_EINVAL, "must not be qkv"),
    (dict(P=100), binding.VLF_EINVAL, "the longest sequence has 156"),
    (dict(scale=float("inf")), binding.VLF_EINVAL, "scale"),
])
def test_rotate_qkv_rejects_bad_arguments_before_launching(kw, status, text):
    rc, msg = _rotate_qkv_status(**kw)
    assert rc == status and text in msg, (rc, msg)


def test_rotate_qkv_with_no_tiles_is_a_no_op():
    assert _rotate_qkv_status(num_tiles=0, dst=None)[0] == binding.VLF_OK
