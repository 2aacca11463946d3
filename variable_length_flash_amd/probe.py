"""ctypes binding of libvlf_probe.so (include/vlf_probe.h): the matrix-unit probe the benchmark
sets the forward's rate against, and the overlap probe that measures how the matrix unit, the
vector unit and LDS operand reads share a SIMD. It is not part of the attention path."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libvlf_probe.so")
EXPORTS = ("vlf_probe_mfma", "vlf_probe_overlap", "vlf_probe_schedule", "vlf_probe_last_error")
FLOP_PER_MFMA = 32 * 32 * 16 * 2  # v_mfma_f32_32x32x16_bf16

_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run python -m "
                               "variable_length_flash_amd.build")
        lib = ctypes.CDLL(LIBRARY)
        lib.vlf_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
        lib.vlf_probe_mfma.restype = ctypes.c_int
        lib.vlf_probe_overlap.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3
        lib.vlf_probe_overlap.restype = ctypes.c_int
        lib.vlf_probe_schedule.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 3
        lib.vlf_probe_schedule.restype = ctypes.c_int
        lib.vlf_probe_last_error.argtypes = []
        lib.vlf_probe_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def mfma_peak(device, iters: int = 20000, reps: int = 3):
    """Sustained bf16 matrix rate and shader clock on ``device``: two four-wave workgroups per
    CU issuing only v_mfma_f32_32x32x16_bf16 on independent accumulators. Returns a dict:
    TFLOP/s of the fastest of ``reps`` launches (HIP events on the launch stream), the clock
    (shader ticks over 100 MHz ticks, median over workgroups), the matrix clocks per
    instruction and SIMD that rate and clock imply, and a workgroup's own loop time (equal to
    the launch's when a CU's workgroups run side by side, half of it when they run in turn)."""
    import torch
    lib = load_library()
    dev = torch.device(device)
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    blocks = 2 * cus
    record = torch.zeros(4 * blocks, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch():
        rc = lib.vlf_probe_mfma(int(iters), int(blocks), record.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(lib.vlf_probe_last_error().decode())

    launch()  # warm-up
    torch.cuda.synchronize(dev)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        torch.cuda.synchronize(dev)
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    rec = record.view(blocks, 4).cpu()
    ticks, real = rec[:, 0].double(), rec[:, 1].double()
    clock = float((ticks / (real / 100e6)).median()) / 1e9
    flop = blocks * 4 * iters * 8 * FLOP_PER_MFMA
    tflops = flop / (best / 1e3) / 1e12
    # matrix clocks per instruction on a SIMD over the whole launch: each SIMD issues
    # blocks * 8 * iters / cus of them in the launch's time at the measured clock
    per_simd = blocks * 8 * iters / cus
    per_mfma = best / 1e3 * clock * 1e9 / per_simd
    wg_ms = float((real / 100e6).median()) * 1e3
    return {"tflops": round(tflops, 1), "clock_ghz": round(clock, 3),
            "clocks_per_mfma": round(per_mfma, 2), "ms": round(best, 4),
            "workgroup_ms_median": round(wg_ms, 4), "cus": cus, "workgroups": blocks,
            "instruction": "v_mfma_f32_32x32x16_bf16"}


ROLES = {0: "idle", 1: "mfma", 2: "exp", 3: "fma", 4: "softmax", 5: "step", 6: "step_lds",
         7: "step_lds_step_ahead", 8: "step_lds_four_ahead", 9: "lds_reads",
         10: "step64_lds_four_ahead"}
# the pairs whose loop times describe the forward's wave step: each role alone (its partner
# idle), then side by side on one SIMD
OVERLAP_PAIRS = ((1, 0), (2, 0), (3, 0), (4, 0), (1, 1), (2, 2), (3, 3), (4, 4), (1, 2), (1, 4),
                 (5, 0), (5, 5), (6, 0), (6, 6), (7, 0), (7, 7), (8, 0), (8, 8), (9, 0), (9, 9), (10, 0), (10, 10))


def overlap(device, pairs=OVERLAP_PAIRS, iters: int = 4000):
    """Loop time of the overlap probe (vlf_probe_overlap) for each (lo, hi) role pair, one
    eight-wave workgroup per CU so that waves 0-3 and 4-7 pair up on the four SIMDs. Returns a
    list of dicts: the roles, shader clocks per iteration from the common start to the last
    wave's end and of each half's own loop (medians over workgroups), and the clock. A role's clocks per iteration alone, against two of it side by
    side and against a pair of different roles, says how far the two units overlap."""
    import torch
    lib = load_library()
    dev = torch.device(device)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(512 * cus, dtype=torch.float32, device=dev)
    record = torch.zeros(4 * cus, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = []
    for lo, hi in pairs:
        for _ in range(2):  # the first launch warms the clock and the code
            rc = lib.vlf_probe_overlap(int(lo), int(hi), int(iters), int(cus), sink.data_ptr(),
                                       record.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(lib.vlf_probe_last_error().decode())
        torch.cuda.synchronize(dev)
        rec = record.view(cus, 4).cpu().double()
        med = [float(rec[:, k].median()) for k in range(4)]
        ghz = float((rec[:, 0] / (rec[:, 1] / 100e6)).median()) / 1e9
        out.append({"lo": ROLES[lo], "hi": ROLES[hi],
                    "clocks_per_iter": round(med[0] / iters, 1),
                    "lo_clocks_per_iter": round(med[2] / iters, 1),
                    "hi_clocks_per_iter": round(med[3] / iters, 1),
                    "clock_ghz": round(ghz, 3)})
    return out


SCHEDULES = {0: ("three groups", 3), 1: ("three groups, softmax phases empty", 3),
             2: ("three groups, products empty", 3), 3: ("four groups", 4),
             4: ("four groups, softmax phases empty", 4), 5: ("four groups, products empty", 4)}


def schedules(device, steps: int = 2000):
    """Shader clocks per 32-row wave step on one SIMD for the phase schedules of
    vlf_probe_schedule (kinds 0-5, medians over one workgroup per CU), and the matrix unit's
    toll on vector work (kinds 6-9): the clocks per iteration of the vector waves without and
    beside a wave of back-to-back MFMAs, and the toll per MFMA that difference implies."""
    import torch
    lib = load_library()
    dev = torch.device(device)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(1024 * cus, dtype=torch.float32, device=dev)
    record = torch.zeros(16 * cus, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(kind):
        for _ in range(2):  # the first launch warms the clock and the code
            rc = lib.vlf_probe_schedule(int(kind), int(steps), int(cus), sink.data_ptr(),
                                        record.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(lib.vlf_probe_last_error().decode())
        torch.cuda.synchronize(dev)
        return record.view(cus, 16).cpu().double()

    rows = []
    for kind, (name, groups) in SCHEDULES.items():
        clocks = float(launch(kind)[:, 0].median()) / (groups * steps)
        rows.append({"schedule": name, "waves_per_simd": groups,
                     "clocks_per_wave_step": round(clocks, 1),
                     "matrix_busy_pct": round(100 * 16 * 32 / clocks, 1)})
    toll = []
    for op, base, with_mfma in (("fma", 6, 7), ("exp", 8, 9)):
        alone = float(launch(base)[:, 4:12].median()) / steps
        rec = launch(with_mfma)
        beside = float(rec[:, 4:12].median()) / steps
        mfma_iter = float(rec[:, :4].median()) / steps  # clocks per four MFMAs
        mfmas = 4 * beside / mfma_iter  # MFMAs issued on the SIMD during one vector iteration
        toll.append({"vector_op": op, "clocks_per_16_alone": round(alone, 1),
                     "clocks_per_16_beside_mfma": round(beside, 1),
                     "mfma_clocks_per_instruction": round(mfma_iter / 4, 1),
                     "toll_clocks_per_mfma": round((beside - alone) / mfmas, 1)})
    return {"schedules": rows, "mfma_toll": toll}
