"""Seeded synthetic inputs for the routed-expert prompt MoE layer.

This module only draws random numbers; it holds none of the layer's arithmetic
(no routing, quantization, matrix products or packing).  Both the CPU oracle's
tests and the HIP path's tests and benchmark take their inputs from here, so the
two sides see bit-identical arrays.

Shapes follow the layer the Strata pages describe (Winery-Strata prefill.cpp
page, the constants at the top of the file: hidden N = 2560, NE = 512 routed
experts, K = 10 per token) with an expert FFN width of I = 1024, plus a tiny
layer for fast checks.  The pages measure on private
prompts and a trained GGUF pack; neither is available, so these seeded
synthetic arrays stand in for them at the same shapes.

Recipe (every stream is a numpy PCG64 generator seeded from a SeedSequence
built from the layer seed and a fixed tag, so any expert can be regenerated on
its own, in any order):

  x      [T][H]   fp32   standard normal drawn in float64, rounded to fp32;
                          stream (seed, 1).
  W_r    [H][E]   fp32   normal, standard deviation 0.05, drawn in float64,
                          rounded to fp32; stream (seed, 2).
  bias   [E]      fp32   only for the skewed layer: perm = permutation(E) on
                          stream (seed, 3); rank = perm + 1;
                          bias = 2.0 * ln(1 / rank**1.2) (Zipf, s = 1.2).
  expert e, matrix m (0 = gate, 1 = up, 2 = down):
         codes    uint8 in {0,1,2,3}, uniform; stream (seed, 100, e, m).
         scales   uniform on [0.005, 0.02] drawn in float64, rounded to fp16
                  (round to nearest even); stream (seed, 200, e, m).
         gate/up codes are [I][H] each (reduction dim H contiguous), stacked
         as [2I][H] with gate rows first; down codes are [H][I].  Scales hold
         one value per 32 consecutive codes along the reduction dim.

Scales are returned as uint16 arrays holding the fp16 bit patterns (the fp16
value is the truth; it is what both sides read).
"""
from __future__ import annotations

import dataclasses

import numpy as np

BLOCK = 32  # values per quantization block along a reduction dimension


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One routed-expert MoE layer workload."""

    name: str
    T: int   # tokens in the chunk
    H: int   # hidden size
    E: int   # routed experts
    K: int   # experts per token
    I: int   # expert FFN width
    skewed: bool = False  # add the Zipf router bias
    fmt: str = "q2_sym"   # weight map label: "q2_sym" or "q2_0" (the pages' own packs)
    shared: bool = False  # add a shared expert (index E) with its scalar gate vector

    @property
    def n(self) -> int:
        return self.T * self.K


# The five layers the layer is checked and measured on.
SHAPES = {
    "tiny": LayerShape("tiny", T=64, H=256, E=16, K=2, I=128),
    "stream_all_1k": LayerShape("stream_all_1k", T=1024, H=2560, E=512, K=10, I=1024),
    "chunk_8k": LayerShape("chunk_8k", T=8192, H=2560, E=512, K=10, I=1024),
    "long_32k": LayerShape("long_32k", T=32768, H=2560, E=512, K=10, I=1024),
    "skewed_4k": LayerShape("skewed_4k", T=4096, H=2560, E=512, K=10, I=1024, skewed=True),
}

# Further workloads of the same layer: the pages' own expert geometry and weight
# map (I = 640, Q2_0) at a 2048-token chunk, and a 256-token chunk.
EXTRA_SHAPES = {
    "pages_q2_0_2k": LayerShape("pages_q2_0_2k", T=2048, H=2560, E=512, K=10, I=640, fmt="q2_0"),
    # a short chunk (about 5 rows per expert): the small-T end of the range
    "short_256": LayerShape("short_256", T=256, H=2560, E=512, K=10, I=1024),
    # a decode-sized window (320 pairs over 512 experts: mostly one row per hit expert)
    "window_32": LayerShape("window_32", T=32, H=2560, E=512, K=10, I=1024),
    # 1.25 and 2.5 rows per expert on average: either side of the GEMV's threshold
    "window_64": LayerShape("window_64", T=64, H=2560, E=512, K=10, I=1024),
    "window_128": LayerShape("window_128", T=128, H=2560, E=512, K=10, I=1024),
    # the MoE half with its shared expert: the 8192-token chunk, and the pages'
    # geometry (there the shared expert has the routed experts' width, 640)
    "chunk_8k_shared": LayerShape("chunk_8k_shared", T=8192, H=2560, E=512, K=10, I=1024, shared=True),
    "pages_shared_2k": LayerShape("pages_shared_2k", T=2048, H=2560, E=512, K=10, I=640, fmt="q2_0", shared=True),
}


def shape(name: str) -> LayerShape:
    return SHAPES[name] if name in SHAPES else EXTRA_SHAPES[name]


def custom(T: int, H: int, E: int, K: int, I: int, skewed: bool = False, fmt: str = "q2_sym",
           shared: bool = False) -> LayerShape:
    """A layer of arbitrary (test) size."""
    name = (f"T{T}_H{H}_E{E}_K{K}_I{I}" + ("_skew" if skewed else "") + ("" if fmt == "q2_sym" else "_" + fmt)
            + ("_shared" if shared else ""))
    return LayerShape(name, T, H, E, K, I, skewed, fmt, shared)


def _rng(*tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(tag))))


def activations(s: LayerShape, seed: int = 0) -> np.ndarray:
    """x [T][H] fp32."""
    return _rng(seed, 1).standard_normal((s.T, s.H)).astype(np.float32)


def router_weight(s: LayerShape, seed: int = 0) -> np.ndarray:
    """W_r [H][E] fp32 (hidden-major: column e is expert e's router vector)."""
    return _rng(seed, 2).normal(0.0, 0.05, (s.H, s.E)).astype(np.float32)


def shared_gate_weight(s: LayerShape, seed: int = 0) -> np.ndarray:
    """The shared expert's scalar gate vector [H] fp32 (drawn like a router
    column).  The shared expert's own arrays are expert(s, s.E, seed)."""
    return _rng(seed, 4).normal(0.0, 0.05, s.H).astype(np.float32)


def router_bias(s: LayerShape, seed: int = 0) -> np.ndarray | None:
    """The skewed layer's per-expert bias [E] fp32, else None."""
    if not s.skewed:
        return None
    perm = _rng(seed, 3).permutation(s.E)
    rank = (perm + 1).astype(np.float64)
    return (2.0 * np.log(1.0 / rank ** 1.2)).astype(np.float32)


def _codes(rows: int, cols: int, *tag: int) -> np.ndarray:
    return _rng(*tag).integers(0, 4, size=(rows, cols), dtype=np.uint8)


def _scales(rows: int, cols: int, *tag: int) -> np.ndarray:
    d = _rng(*tag).uniform(0.005, 0.02, size=(rows, cols // BLOCK))
    return d.astype(np.float16).view(np.uint16)


@dataclasses.dataclass
class Expert:
    """Canonical arrays of one expert."""

    codes_gu: np.ndarray   # uint8 [2I][H]: gate rows 0..I-1, up rows I..2I-1
    scales_gu: np.ndarray  # uint16 (fp16 bits) [2I][H/32]
    codes_d: np.ndarray    # uint8 [H][I]
    scales_d: np.ndarray   # uint16 (fp16 bits) [H][I/32]


def expert(s: LayerShape, e: int, seed: int = 0) -> Expert:
    gate_c = _codes(s.I, s.H, seed, 100, e, 0)
    up_c = _codes(s.I, s.H, seed, 100, e, 1)
    down_c = _codes(s.H, s.I, seed, 100, e, 2)
    gate_s = _scales(s.I, s.H, seed, 200, e, 0)
    up_s = _scales(s.I, s.H, seed, 200, e, 1)
    down_s = _scales(s.H, s.I, seed, 200, e, 2)
    return Expert(np.concatenate([gate_c, up_c]), np.concatenate([gate_s, up_s]), down_c, down_s)


def experts(s: LayerShape, e0: int, e1: int, seed: int = 0) -> Expert:
    """Experts [e0, e1) stacked along a new leading axis."""
    parts = [expert(s, e, seed) for e in range(e0, e1)]
    return Expert(
        np.stack([p.codes_gu for p in parts]),
        np.stack([p.scales_gu for p in parts]),
        np.stack([p.codes_d for p in parts]),
        np.stack([p.scales_d for p in parts]),
    )
