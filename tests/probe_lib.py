"""Loader for the test-only conversion probe library
(tests/gpu_probe/libnvfp4_probe.so, built by block_scaled_fp4_nibble_amd.build).

Its kernels run the product's device conversion helpers over exhaustive input
sets; the tests compare the results with the oracle."""
from __future__ import annotations

import ctypes
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_probe",
                     "libnvfp4_probe.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise OSError("probe library not built: %s (run block_scaled_fp4_nibble_amd.build)"
                          % _PATH)
        lib = ctypes.CDLL(_PATH)
        P, U32, I = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
        lib.probe_e2m1_pack.argtypes = [U32, U32, P, P]
        lib.probe_e4m3_encode.argtypes = [U32, U32, P, P]
        lib.probe_e4m3_decode.argtypes = [P, P]
        lib.probe_quotient.argtypes = [P, P, P, U32, P]
        lib.probe_dequant.argtypes = [P, U32, P, P]
        for f in ("probe_e2m1_pack", "probe_e4m3_encode", "probe_e4m3_decode", "probe_quotient",
                  "probe_dequant"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())
