"""ctypes binding of libstrata_probe: matrix-unit measurements (not part of
the layer).  Each function mirrors the C entry point of the same name in
csrc/probe.hip."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstrata_probe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
_lib = ctypes.CDLL(LIB_PATH)
_d = ctypes.POINTER(ctypes.c_double)
_f = ctypes.POINTER(ctypes.c_float)
_lib.strata_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _d, _d]
_lib.strata_probe_scaled_blocks.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _d, _d]
_lib.strata_probe_scaled_tiles.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _d, _d]
_lib.strata_probe_block_step.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _d, _d]
_lib.strata_probe_mfma_f16.argtypes = [_f, _f, _f, _f]
_lib.strata_probe_hbm_read.argtypes = [ctypes.c_int64, ctypes.c_int32, _d, _d]

# MFMA forms of strata_probe_mfma_rate, by index
KINDS = ["f16_16x16x32", "f16_32x32x16", "i8_16x16x64", "i8_32x32x32", "i8_16x16x32", "i8_32x32x16"]


def strata_probe_mfma_rate(kind: str, groups: int = 4096, iters: int = 512) -> tuple[float, float]:
    """(ops per second, kernel ms) of one MFMA form at full occupancy."""
    r, ms = ctypes.c_double(), ctypes.c_double()
    rc = _lib.strata_probe_mfma_rate(KINDS.index(kind), groups, iters, ctypes.byref(r), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"strata_probe_mfma_rate failed ({rc})")
    return r.value, ms.value


def strata_probe_scaled_blocks(int8: bool, groups: int = 4096, blocks: int = 512) -> tuple[float, float]:
    """(scaled output-blocks per second, kernel ms) of the fp16 (layer) or int8 formulation."""
    r, ms = ctypes.c_double(), ctypes.c_double()
    rc = _lib.strata_probe_scaled_blocks(int(int8), groups, blocks, ctypes.byref(r), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"strata_probe_scaled_blocks failed ({rc})")
    return r.value, ms.value


def strata_probe_scaled_tiles(form: str, tiles: int, groups: int = 2048, blocks: int = 512) -> tuple[float, float]:
    """(scaled output-blocks per second, kernel ms) of the fp16 form at `tiles` (1 or 6) output tiles of
    32 x 32 per wave and block; form "16x16x32" (the layer's MFMA) or "32x32x16"."""
    r, ms = ctypes.c_double(), ctypes.c_double()
    rc = _lib.strata_probe_scaled_tiles(["16x16x32", "32x32x16"].index(form), tiles, groups, blocks,
                                        ctypes.byref(r), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"strata_probe_scaled_tiles failed ({rc})")
    return r.value, ms.value


def strata_probe_block_step(step: int, groups: int = 2048, blocks: int = 512) -> tuple[float, float]:
    """(scaled output-blocks per second, kernel ms) of the gate/up block step built up: 0 the products and
    FMAs with activation loads, 1 plus the unpack stand-in and the LDS exchange with a barrier per block,
    2 the same with a barrier per two blocks."""
    r, ms = ctypes.c_double(), ctypes.c_double()
    rc = _lib.strata_probe_block_step(step, groups, blocks, ctypes.byref(r), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"strata_probe_block_step failed ({rc})")
    return r.value, ms.value


def strata_probe_hbm_read(nbytes: int = 2 << 30, groups: int = 4096) -> tuple[float, float]:
    """(GB/s, kernel ms) of a plain streaming read of nbytes from HBM."""
    r, ms = ctypes.c_double(), ctypes.c_double()
    rc = _lib.strata_probe_hbm_read(nbytes, groups, ctypes.byref(r), ctypes.byref(ms))
    if rc != 0:
        raise RuntimeError(f"strata_probe_hbm_read failed ({rc})")
    return r.value, ms.value


def strata_probe_mfma_f16(A, B, C) -> np.ndarray:
    """D = A B + C by one v_mfma_f32_16x16x32_f16 (A [16][32] and B [32][16] rounded to fp16)."""
    A = np.ascontiguousarray(A, np.float32)
    B = np.ascontiguousarray(B, np.float32)
    C = np.ascontiguousarray(C, np.float32)
    assert A.shape == (16, 32) and B.shape == (32, 16) and C.shape == (16, 16)
    D = np.empty((16, 16), np.float32)
    p = lambda a: a.ctypes.data_as(_f)  # noqa: E731
    rc = _lib.strata_probe_mfma_f16(p(A), p(B), p(C), p(D))
    if rc != 0:
        raise RuntimeError(f"strata_probe_mfma_f16 failed ({rc})")
    return D
