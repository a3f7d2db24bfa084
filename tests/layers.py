"""Test helpers: seeded layers on the GPU and oracle references, cached per
session (the four full-size layers share one set of 512 experts)."""
from __future__ import annotations

import numpy as np

import oracle
import synthetic as S

_expert_cache: dict = {}
_gpu_experts: dict = {}


def canonical_expert(s: S.LayerShape, e: int, seed: int = 0):
    key = (s.H, s.I, seed, e)
    ex = _expert_cache.get(key)
    if ex is None:
        ex = S.expert(s, e, seed)
        _expert_cache[key] = ex
    return ex


def getter(s: S.LayerShape, seed: int = 0):
    return lambda e: canonical_expert(s, e, seed)


def gpu_experts(s: S.LayerShape, seed: int = 0, chunk: int = 32):
    """Packed experts of the layer on cuda, with the layer's router bias."""
    import torch

    import quantized_routed_expert_logits_amd as qm

    key = (s.E, s.H, s.I, seed, s.fmt, s.shared)
    base = _gpu_experts.get(key)
    nb = s.E + s.shared  # the shared expert's blob is the last one
    if base is None:
        base = qm.Experts(s.E, s.H, s.I, device="cuda", fmt=s.fmt, shared=s.shared)
        for e0 in range(0, nb, chunk):
            e1 = min(nb, e0 + chunk)
            parts = [canonical_expert(s, e, seed) for e in range(e0, e1)]
            base.pack(e0, np.stack([p.codes_gu for p in parts]), np.stack([p.scales_gu for p in parts]),
                      np.stack([p.codes_d for p in parts]), np.stack([p.scales_d for p in parts]))
        torch.cuda.synchronize()
        _gpu_experts[key] = base
    if s.shared:
        base = base.with_shared_gate(torch.from_numpy(S.shared_gate_weight(s, seed)).cuda())
    bias = S.router_bias(s, seed)
    return base.with_router_bias(None if bias is None else torch.from_numpy(bias).cuda())


def shared_args(s: S.LayerShape, seed: int = 0):
    """The oracle's shared-expert argument for the layer (None without one)."""
    return (canonical_expert(s, s.E, seed), S.shared_gate_weight(s, seed)) if s.shared else None


def gate_bound(x, wg) -> np.ndarray:
    """Per-token bound of |g_gpu - g| for the fp32 gate: the dot of H products
    in fp32 is within (H + 6) 2^-24 sum|x w| of the exact one, sigmoid's slope
    is at most 1/4, and exp, add and divide add a few units of 2^-24."""
    H = x.shape[1]
    return 0.25 * (H + 6) * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(wg.astype(np.float64))) + 8 * 2.0 ** -24


def check_h_codes(q_gpu, s_gpu, h_ref, q_ref, s_ref, tie_tol=2e-3):
    """SwiGLU-output codes: the GPU rounds its fp32 h, the oracle RN32 of an
    exact h, so a code may differ only where the oracle's quotient is within
    tie_tol of a rounding boundary, and then by one.  Returns the mismatch
    rate."""
    q_gpu = np.asarray(q_gpu, np.int32)
    q_ref = np.asarray(q_ref, np.int32)
    s_gpu = np.asarray(s_gpu, np.float64)
    s_ref = np.asarray(s_ref, np.float64)
    nz = s_ref > 0
    assert np.all(s_gpu[~nz] == 0)
    rel = np.abs(s_gpu[nz] / s_ref[nz] - 1.0)
    assert rel.max(initial=0.0) <= 1e-5, f"H scales differ by {rel.max():.2e}"
    diff = q_gpu != q_ref
    if diff.any():
        rows, cols = np.nonzero(diff)
        sr = np.repeat(s_ref, 32, axis=1)[rows, cols]
        t = np.abs(h_ref[rows, cols]) / sr
        frac = t - np.floor(t)
        assert np.all(np.abs(frac - 0.5) < tie_tol), "an H code differs away from a rounding tie"
        assert np.all(np.abs(q_gpu[rows, cols] - q_ref[rows, cols]) == 1)
    return diff.mean()


def rel_err(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-300))


def down_error_bound(s: S.LayerShape, ref: dict, seed: int = 0) -> np.ndarray:
    """Per-output bound of |y_gpu - y| for the down GEMM and the combine.

    The down GEMM takes each block's sum of (q - 1) d times the int8 H codes
    exactly (an integer times an fp16 d, within fp32's 24 bits), then adds it
    times the block's H scale with one fp32 FMA; the offset term of the
    symmetric map adds sum_b d u_b with u split into two fp16 halves (22
    bits); the routing-weight product and the K-term combine round in fp32 as
    well.  The GEMV kernel (chunks of one or two rows) takes the int32 block
    sum times the block's H scale and then times d: two roundings per block.
    Every rounding is relative to at most the sum of absolute terms, and
    there are fewer than 2 I / 32 + K + 8 of them on any output's path, so
        |dy[t, j]| <= (2 I / 32 + K + 8) 2^-23 * sum_k p[t,k] sum_i |W_e[j,i]| |h[t,k,i]|.
    The absolute weights come from the codes and fp16 scales directly."""
    n = s.T * s.K
    h_abs = np.abs(ref["qh"].astype(np.float64) * np.repeat(ref["sh"].astype(np.float64), 32, axis=1))
    bound = np.zeros((s.T, s.H))
    off, src, slot = ref["offsets"], ref["src"], ref["slot"]
    p = ref["p"].reshape(-1)
    inv = np.empty(n, np.int64)  # grouped row g holds routed pair inv[g]: token src[g], weight p at that pair
    inv[slot] = np.arange(n)
    for e in range(s.E):
        o0, o1 = off[e], off[e + 1]
        if o1 == o0:
            continue
        ex = canonical_expert(s, e, seed)
        d = ex.scales_d.view(np.float16).astype(np.float64)
        w_abs = np.abs(np.repeat(d, 32, axis=1) * (ex.codes_d.astype(np.float64) - oracle.code_zero(s.fmt)))
        contrib = h_abs[o0:o1] @ w_abs.T                      # [rows][H]
        pairs = inv[o0:o1]
        np.add.at(bound, src[o0:o1], contrib * p[pairs][:, None])
    return (2 * s.I / 32 + s.K + 8) * 2.0 ** -23 * bound
