"""ctypes binding of libbha_probe.so, the HBM streaming probe (include/bha_probe.h).

Argument marshalling only. ``stream_gbps`` allocates the buffers, runs
launches of the probe on rotating regions of a source buffer (so that no launch
finds its bytes in the Infinity Cache from the previous one) and returns the
bandwidth of the median launch, timed with HIP events on the launch stream.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbha_probe.so")
_lib = None


class bha_probe_cfg(ctypes.Structure):
    _fields_ = [("loads_per_lane", ctypes.c_int32), ("buffers", ctypes.c_int32), ("nontemporal", ctypes.c_int32),
                ("wgs_per_cu", ctypes.c_int32), ("store_kb_per_wave", ctypes.c_int32), ("store_mode", ctypes.c_int32)]


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m linear_attention_block_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        C = ctypes.POINTER(bha_probe_cfg)
        for name in ("bha_probe_trip_read_bytes", "bha_probe_trip_write_bytes", "bha_probe_sink_floats"):
            getattr(lib, name).argtypes = [C]
            getattr(lib, name).restype = ctypes.c_int64
        lib.bha_probe_stream.argtypes = [C, P, ctypes.c_int64, P, P, P]
        lib.bha_probe_stream.restype = ctypes.c_int
        _lib = lib
    return _lib


def cfg(loads_per_lane=16, buffers=1, nontemporal=1, wgs_per_cu=2, store_kb_per_wave=0, store_mode=0):
    return bha_probe_cfg(loads_per_lane, buffers, nontemporal, wgs_per_cu, store_kb_per_wave, store_mode)


def stream_gbps(c: bha_probe_cfg, read_bytes: int, launches: int = 10, regions: int = 5, device=None):
    """Run the probe over about ``read_bytes`` per launch; returns
    (read + written bytes per launch, median launch seconds, GB/s)."""
    import numpy as np
    import torch

    lib = load_library()
    dev = device or torch.device("cuda:0")
    rb = lib.bha_probe_trip_read_bytes(ctypes.byref(c))
    wb = lib.bha_probe_trip_write_bytes(ctypes.byref(c))
    nsink = lib.bha_probe_sink_floats(ctypes.byref(c))
    if rb <= 0 or wb < 0 or nsink <= 0:
        raise ValueError("invalid probe configuration")
    trips = max(1, read_bytes // rb)
    src = torch.ones(regions * trips * rb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty(max(1, regions * trips * wb // 4), dtype=torch.float32, device=dev)
    sink = torch.empty(nsink, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(i):
        sp = src.data_ptr() + (i % regions) * trips * rb
        dp = dst.data_ptr() + (i % regions) * trips * wb
        st = lib.bha_probe_stream(ctypes.byref(c), ctypes.c_void_p(sp), trips, ctypes.c_void_p(dp),
                                  ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"bha_probe_stream failed with status {st}")

    for i in range(regions):
        run(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        run(i)
        e1.record(stream)
    torch.cuda.synchronize(dev)
    t = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3
    moved = trips * (rb + wb)
    del src, dst, sink
    return moved, t, moved / t / 1e9
