"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something it does not compute itself:
numpy/IEEE library routines, an independent dense formulation, closed forms,
invariants, exhaustive round-trips and hand-worked fixtures under
tests/golden/.  The cases are chosen so that a plausible slip anywhere in the
oracle (a dropped offset, a sign, a transposed operand, a wrong tie rule, an
unstable sort, half-even instead of half-away rounding) fails at least one.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synthetic as S
from conftest import GOLDEN

RNG = np.random.default_rng(1234)


def _read_golden(name):
    lines = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                lines.append(line.split())
    return lines


# ------------------------------------------------------------------- formats
def test_half_decoding_matches_ieee_for_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_dequant_round_trip_exact():
    """w = d*(q - 1.5) is exact in fp32 and (w / d) + 1.5 recovers q exactly."""
    ex = S.expert(S.shape("tiny"), 3)
    d = ex.scales_gu.view(np.float16).astype(np.float64)
    q = ex.codes_gu.astype(np.float64).reshape(d.shape[0], d.shape[1], 32)
    w = d[:, :, None] * (q - 1.5)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    assert np.array_equal(w / d[:, :, None] + 1.5, q)


# -------------------------------------------------------------- c1 router
def test_router_logits_match_dense_float64():
    s = S.custom(T=37, H=320, E=24, K=3, I=64)
    x = S.activations(s, 5)
    wr = S.router_weight(s, 5)
    got = oracle.router_logits(x, wr)
    ref = x.astype(np.float64) @ wr.astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_router_logits_are_the_correctly_rounded_sum():
    s = S.custom(T=6, H=2560, E=8, K=2, I=32)
    x = S.activations(s, 9)
    wr = S.router_weight(s, 9)
    got = oracle.router_logits(x, wr)
    for t in range(s.T):
        for e in range(s.E):
            exact = math.fsum(float(a) * float(b) for a, b in zip(x[t], wr[:, e]))
            assert abs(got[t, e] - exact) <= 2 * abs(exact) * 2.0 ** -53 + 1e-300


def test_router_bias_is_added():
    s = S.shape("tiny")
    x, wr = S.activations(s), S.router_weight(s)
    bias = np.linspace(-3, 3, s.E).astype(np.float32)
    a = oracle.router_logits(x, wr)
    b = oracle.router_logits(x, wr, bias)
    assert np.allclose(b - a, bias.astype(np.float64)[None, :], rtol=0, atol=1e-12)


def test_skewed_bias_is_zipf_over_a_permutation():
    s = S.shape("skewed_4k")
    b = S.router_bias(s).astype(np.float64)
    rank = np.exp(-b / 2.4)  # bias = -2.4 ln(rank)
    assert np.allclose(np.sort(rank), np.arange(1, s.E + 1), rtol=1e-5)


# ---------------------------------------------------------- c2 top-K/softmax
def test_topk_matches_stable_argsort_and_softmax():
    s = S.custom(T=50, H=64, E=40, K=7, I=32)
    logits = RNG.standard_normal((s.T, s.E))
    logits[:, 5] = logits[:, 9]  # exact ties
    ids, p = oracle.topk_softmax(logits, s.K)
    ref_ids = np.argsort(-logits, axis=1, kind="stable")[:, : s.K]
    assert np.array_equal(ids, ref_ids)
    sel = np.take_along_axis(logits, ref_ids, 1)
    full = np.exp(logits - logits.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    ref_p = np.take_along_axis(full, ref_ids, 1)
    ref_p /= ref_p.sum(1, keepdims=True)
    assert np.abs(p - ref_p).max() < 1e-14
    assert np.abs(p.sum(1) - 1).max() < 1e-14
    assert np.all(np.diff(sel, axis=1) <= 0) and np.all(np.diff(p, axis=1) <= 1e-15)


def test_topk_golden_hand_example():
    g = _read_golden("route_tiny.txt")
    vals = {row[0]: row[1:] for row in g}
    logits = np.array([[float(v) for v in vals["logits"]]])
    K = int(vals["K"][0])
    ids, p = oracle.topk_softmax(logits, K)
    assert ids[0].tolist() == [int(v) for v in vals["ids"]]
    assert np.allclose(p[0], [float(v) for v in vals["p"]], rtol=0, atol=1e-16)


def test_zero_router_gives_first_k_with_equal_weights():
    s = S.custom(T=5, H=64, E=12, K=4, I=32)
    x = S.activations(s)
    ids, p = oracle.topk_softmax(oracle.router_logits(x, np.zeros((s.H, s.E), np.float32)), s.K)
    assert np.array_equal(ids, np.tile(np.arange(s.K), (s.T, 1)))
    assert np.allclose(p, 1.0 / s.K, rtol=0, atol=1e-15)


def test_duplicate_router_columns_tie_to_lower_index():
    s = S.custom(T=40, H=64, E=10, K=10, I=32)
    x = S.activations(s, 2)
    wr = S.router_weight(s, 2)
    wr[:, 7] = wr[:, 2]
    ids, p = oracle.topk_softmax(oracle.router_logits(x, wr), s.K)
    pos = {int(e): k for k, e in enumerate(ids[0])}
    for t in range(s.T):
        row = ids[t].tolist()
        assert row.index(2) + 1 == row.index(7)  # adjacent, lower index first
        assert p[t, row.index(2)] == p[t, row.index(7)]
    assert pos


def test_k1_weight_is_one():
    logits = RNG.standard_normal((9, 5))
    ids, p = oracle.topk_softmax(logits, 1)
    assert np.array_equal(ids[:, 0], logits.argmax(1)) and np.all(p == 1.0)


# ------------------------------------------------------------- c3 grouping
def _check_grouping(ids, E, offsets, src, slot):
    T, K = ids.shape
    n = T * K
    flat = ids.reshape(-1)
    cnt = np.bincount(flat, minlength=E)
    assert offsets[0] == 0 and offsets[E] == n
    assert np.array_equal(np.diff(offsets), cnt)
    assert np.array_equal(np.bincount(src, minlength=T), np.full(T, K))
    for e in range(E):
        g = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(g) > 0)  # sorted, and a token at most once per expert
    assert np.array_equal(np.sort(slot), np.arange(n))
    assert np.array_equal(src[slot], np.arange(n) // K)
    rows_expert = np.repeat(np.arange(E), cnt)
    assert np.array_equal(rows_expert[slot], flat)


def test_grouping_invariants_and_stable_sort():
    for T, E, K in [(64, 16, 2), (333, 37, 5), (1000, 512, 10)]:
        logits = RNG.standard_normal((T, E))
        ids, _ = oracle.topk_softmax(logits, K)
        offsets, src, slot = oracle.group(ids, E)
        _check_grouping(ids, E, offsets, src, slot)
        order = np.argsort(ids.reshape(-1), kind="stable")
        assert np.array_equal(src, order // K)
        assert np.array_equal(slot[order], np.arange(T * K))


def test_grouping_with_empty_experts_and_skew():
    T, E, K = 200, 64, 4
    logits = RNG.standard_normal((T, E))
    logits[:, :6] += 50.0  # experts 0..5 take nearly everything
    ids, _ = oracle.topk_softmax(logits, K)
    offsets, src, slot = oracle.group(ids, E)
    _check_grouping(ids, E, offsets, src, slot)
    assert (np.diff(offsets) == 0).sum() > 40


def test_grouping_rejects_out_of_range_ids():
    ids = np.array([[0, 1], [2, 16]], np.int32)
    with pytest.raises(ValueError):
        oracle.group(ids, 16)
    with pytest.raises(ValueError):
        oracle.group(np.array([[0, -1]], np.int32), 16)


# ------------------------------------------------------------ c4 quantize
def test_quantize_golden_block():
    g = _read_golden("quantize_block.txt")
    scale = float(g[0][1])
    v = np.array([[float(r[0]) for r in g[1:]]], np.float32)
    want = np.array([int(r[1]) for r in g[1:]])
    q, s = oracle.quantize(v)
    assert s[0, 0] == np.float32(scale)
    assert np.array_equal(q[0], want)


def test_quantize_matches_native_fp32_arithmetic():
    """The oracle emulates the fp32 decision in double; numpy float32 division
    is IEEE round-to-nearest, so both must agree bit for bit."""
    v = (RNG.standard_normal((400, 256)) * RNG.choice([1e-3, 1.0, 50.0], (400, 1))).astype(np.float32)
    # plant exact half-way quotients: a block whose max is 127 has s == 1
    v[0, :32] = np.float32(np.arange(32) - 15.5)
    v[0, 0] = 127.0
    q, s = oracle.quantize(v)
    blocks = v.reshape(400, 8, 32)
    a = np.abs(blocks).max(2)
    s_ref = (a / np.float32(127.0)).astype(np.float32)
    assert np.array_equal(s, s_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (blocks / s_ref[:, :, None]).astype(np.float32)
    r = np.where(t >= 0, np.floor(t.astype(np.float64) + 0.5), -np.floor(-t.astype(np.float64) + 0.5))
    r = np.clip(np.nan_to_num(r), -127, 127)
    assert np.array_equal(q.reshape(400, 8, 32), r.astype(np.int8))
    assert np.all(np.abs(q.reshape(400, 8, 32)).max(2) == 127)  # the max element maps to 127


def test_quantize_closed_forms():
    const = np.full((3, 32), 0, np.float32)
    const[0] = 3.25
    const[1] = -0.001
    q, s = oracle.quantize(const)
    assert np.all(q[0] == 127) and s[0, 0] == np.float32(np.float32(3.25) / np.float32(127))
    assert np.all(q[1] == -127)
    assert np.all(q[2] == 0) and s[2, 0] == 0.0


def test_quantize_round_trip_exhaustive():
    """Every code survives q -> q*s -> quantize for several scales."""
    for s_target in [1.0, 0.015625, 0.37, 1e-3, 7.9]:
        codes = np.arange(-127, 128)
        v = np.zeros((len(codes), 32), np.float32)
        v[:, 0] = np.float32(127 * s_target)
        v[:, 1] = (codes * np.float32(s_target)).astype(np.float32)
        q, s = oracle.quantize(v)
        assert np.all(s[:, 0] == s[0, 0])
        ss = np.float64(s[0, 0])
        back = (codes * np.float32(s[0, 0])).astype(np.float32)
        v[:, 1] = back
        q, s = oracle.quantize(v)
        assert np.array_equal(q[:, 1], codes), s_target
        assert abs(ss - s_target) <= 1e-6 * s_target


def test_quantize_error_bound():
    v = RNG.standard_normal((100, 128)).astype(np.float32)
    q, s = oracle.quantize(v)
    rec = q.reshape(100, 4, 32).astype(np.float64) * s[:, :, None]
    err = np.abs(rec - v.reshape(100, 4, 32))
    assert np.all(err <= s[:, :, None] * (0.5 + 1e-6))


# ------------------------------------------------------ c5..c8 experts, combine
# the 2-bit maps: w = d * (q - 1.5) (symmetric) and the pages' Q2_0 packs'
# w = d * (q - 1) (Strata compare page, moe_fused.hpp header comment)
ZERO = {"q2_sym": 1.5, "q2_0": 1.0}


def _dense(ex, fmt="q2_sym"):
    """Independent dense dequantization: W = d * (q - z) as float64 matrices."""
    z = ZERO[fmt]
    I2, H = ex.codes_gu.shape
    d_gu = np.repeat(ex.scales_gu.view(np.float16).astype(np.float64), 32, axis=1)
    W_gu = d_gu * (ex.codes_gu.astype(np.float64) - z)
    d_d = np.repeat(ex.scales_d.view(np.float16).astype(np.float64), 32, axis=1)
    W_d = d_d * (ex.codes_d.astype(np.float64) - z)
    return W_gu[: I2 // 2], W_gu[I2 // 2:], W_d


@pytest.mark.parametrize("fmt", ["q2_sym", "q2_0"])
def test_expert_rows_match_dense_brute_force(fmt):
    for s in [S.shape("tiny"), S.custom(T=4, H=64, E=4, K=2, I=32), S.custom(T=3, H=96, E=2, K=1, I=160)]:
        ex = S.expert(s, 1, seed=7)
        x = S.activations(s, 7)
        qx, sx = oracle.quantize(x)
        h, qh, sh, D = oracle.expert_rows(ex, qx, sx, want_h=True, fmt=fmt)
        Wg, Wu, Wd = _dense(ex, fmt)
        xd = qx.astype(np.float64) * np.repeat(sx.astype(np.float64), 32, axis=1)
        G, U = xd @ Wg.T, xd @ Wu.T
        h_ref = G / (1 + np.exp(-G)) * U
        assert np.abs(h - h_ref).max() <= 1e-12 * np.abs(h_ref).max()
        q_ref, s_ref = oracle.quantize(h.astype(np.float32))  # c6 is c4 on RN32(h)
        assert np.array_equal(qh, q_ref) and np.array_equal(sh, s_ref)
        hd = qh.astype(np.float64) * np.repeat(sh.astype(np.float64), 32, axis=1)
        D_ref = hd @ Wd.T
        assert np.abs(D - D_ref).max() <= 1e-12 * np.abs(D_ref).max()


def test_silu_of_zero_and_zero_input():
    s = S.custom(T=3, H=64, E=2, K=1, I=32)
    ex = S.expert(s, 0)
    qx = np.zeros((3, 64), np.int8)
    sx = np.zeros((3, 2), np.float32)
    h, qh, sh, D = oracle.expert_rows(ex, qx, sx, want_h=True)
    assert np.all(h == 0) and np.all(qh == 0) and np.all(sh == 0) and np.all(D == 0)


def _layer_dense(x, wr, bias, exps, K, fmt="q2_sym"):
    """Fully independent numpy layer: dense weights, per-token loop."""
    logits = x.astype(np.float64) @ wr.astype(np.float64)
    if bias is not None:
        logits = logits + bias.astype(np.float64)
    T, H = x.shape
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(logits, ids, 1)
    w = np.exp(sel - sel[:, :1])
    p = w / w.sum(1, keepdims=True)
    qx, sx = oracle.quantize(x)
    xd = qx.astype(np.float64) * np.repeat(sx.astype(np.float64), 32, axis=1)
    dense = [_dense(ex, fmt) for ex in exps]
    y = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            y[t] += p[t, k] * _ffn_dense(dense[ids[t, k]], xd[t])
    return ids, p, y


def _ffn_dense(W, xdt):
    """One token through one expert with dense weights: SwiGLU, H rounded to
    int8 per 32 (c4 on the fp32-rounded h), down."""
    Wg, Wu, Wd = W
    G, U = Wg @ xdt, Wu @ xdt
    hq, hs = oracle.quantize((G / (1 + np.exp(-G)) * U).astype(np.float32)[None, :])
    hd = hq[0].astype(np.float64) * np.repeat(hs[0].astype(np.float64), 32)
    return Wd @ hd


def test_shared_gate_closed_forms():
    H = 64
    x = S.activations(S.custom(T=5, H=H, E=2, K=1, I=32), 3)
    assert np.all(oracle.shared_gate(x, np.zeros(H, np.float32)) == 0.5)  # sigmoid(0)
    wg = np.zeros(H, np.float32)
    wg[7] = 1.0
    xs = np.zeros((4, H), np.float32)
    xs[:, 7] = [np.log(3.0), -np.log(3.0), 40.0, -40.0]
    g = oracle.shared_gate(xs, wg)
    l3 = float(np.float32(np.log(3.0)))
    assert abs(g[0] - 1.0 / (1.0 + np.exp(-l3))) < 1e-15 and abs(g[0] - 0.75) < 1e-7
    assert abs(g[0] + g[1] - 1.0) < 1e-15  # sigmoid(-s) = 1 - sigmoid(s)
    assert g[2] == 1.0 and 0 < g[3] < 1e-17  # sigmoid(40) rounds to 1 in double; sigmoid(-40) = 4.2e-18
    # the gate is the sigmoid of the plain dot product
    wr = S.shared_gate_weight(S.custom(T=5, H=H, E=2, K=1, I=32))
    dot = x.astype(np.float64) @ wr.astype(np.float64)
    assert np.abs(oracle.shared_gate(x, wr) - 1 / (1 + np.exp(-dot))).max() < 1e-15


@pytest.mark.parametrize("fmt", ["q2_sym", "q2_0"])
def test_layer_with_shared_expert_matches_independent_dense_layer(fmt):
    s = S.custom(T=20, H=96, E=6, K=3, I=64, fmt=fmt, shared=True)
    x, wr = S.activations(s), S.router_weight(s)
    exps = [S.expert(s, e) for e in range(s.E + 1)]
    wg = S.shared_gate_weight(s)
    out = oracle.layer(x, wr, None, lambda e: exps[e], s.E, s.K, fmt=fmt, shared=(exps[s.E], wg))
    ids, p, y = _layer_dense(x, wr, None, exps[: s.E], s.K, fmt)
    qx, sx = oracle.quantize(x)
    xd = qx.astype(np.float64) * np.repeat(sx.astype(np.float64), 32, axis=1)
    W = _dense(exps[s.E], fmt)
    g = 1 / (1 + np.exp(-(x.astype(np.float64) @ wg.astype(np.float64))))
    for t in range(s.T):
        y[t] += g[t] * _ffn_dense(W, xd[t])
    assert np.array_equal(out["ids"], ids)
    assert np.abs(out["shared"]["g"] - g).max() < 1e-14
    assert np.abs(out["y"] - y).max() <= 1e-10 * np.abs(y).max()
    # the sampled-token form gives the same rows
    tok = np.array([0, 7, 19])
    lt = oracle.layer_tokens(x, wr, None, lambda e: exps[e], s.K, tok, fmt=fmt, shared=(exps[s.E], wg))
    assert np.abs(lt["y"] - out["y"][tok]).max() <= 1e-12 * np.abs(y).max()


def test_shared_expert_with_zero_gate_vector_adds_half_its_output():
    s = S.custom(T=9, H=64, E=4, K=2, I=32, shared=True)
    x, wr = S.activations(s), S.router_weight(s)
    exps = [S.expert(s, e) for e in range(s.E + 1)]
    base = oracle.layer(x, wr, None, lambda e: exps[e], s.E, s.K)
    out = oracle.layer(x, wr, None, lambda e: exps[e], s.E, s.K, shared=(exps[s.E], np.zeros(s.H, np.float32)))
    _, _, _, D = oracle.expert_rows(exps[s.E], *oracle.quantize(x))
    assert np.abs(out["y"] - (base["y"] + 0.5 * D)).max() <= 1e-14 * np.abs(out["y"]).max()


@pytest.mark.parametrize("skewed,fmt", [(False, "q2_sym"), (True, "q2_sym"), (False, "q2_0")])
def test_layer_matches_independent_dense_layer(skewed, fmt):
    s = S.custom(T=24, H=96, E=6, K=3, I=64, skewed=skewed, fmt=fmt)
    x, wr, bias = S.activations(s), S.router_weight(s), S.router_bias(s)
    exps = [S.expert(s, e) for e in range(s.E)]
    out = oracle.layer(x, wr, bias, lambda e: exps[e], s.E, s.K, fmt=s.fmt)
    ids, p, y = _layer_dense(x, wr, bias, exps, s.K, fmt)
    assert np.array_equal(out["ids"], ids)
    assert np.abs(out["p"] - p).max() < 1e-14
    assert np.abs(out["y"] - y).max() <= 1e-10 * np.abs(y).max()


def test_single_expert_layer_is_a_plain_quantized_ffn():
    s = S.custom(T=10, H=64, E=1, K=1, I=96)
    x, wr = S.activations(s), S.router_weight(s)
    ex = S.expert(s, 0)
    out = oracle.layer(x, wr, None, lambda e: ex, 1, 1)
    assert np.all(out["p"] == 1.0) and np.all(out["ids"] == 0)
    _, _, _, D = oracle.expert_rows(ex, *oracle.quantize(x))
    assert np.array_equal(out["y"], D)


def test_identical_experts_combine_to_one_expert():
    s = S.custom(T=12, H=64, E=5, K=3, I=32)
    x, wr = S.activations(s), S.router_weight(s)
    ex = S.expert(s, 0)
    out = oracle.layer(x, wr, None, lambda e: ex, s.E, s.K)
    _, _, _, D = oracle.expert_rows(ex, *oracle.quantize(x))
    assert np.abs(out["y"] - D).max() <= 1e-14 * np.abs(D).max()


def test_zero_input_gives_zero_output():
    s = S.custom(T=8, H=64, E=4, K=2, I=32)
    out = oracle.layer(np.zeros((s.T, s.H), np.float32), S.router_weight(s), None,
                       lambda e: S.expert(s, e), s.E, s.K)
    assert np.all(out["y"] == 0)


def test_sampled_tokens_equal_full_layer():
    s = S.custom(T=40, H=64, E=8, K=3, I=32)
    x, wr = S.activations(s), S.router_weight(s)
    get = lambda e: S.expert(s, e)
    full = oracle.layer(x, wr, None, get, s.E, s.K)
    toks = [0, 7, 39, 13]
    part = oracle.layer_tokens(x, wr, None, get, s.K, toks)
    assert np.array_equal(part["ids"], full["ids"][toks])
    assert np.array_equal(part["y"], full["y"][toks])
    rows = full["slot"].reshape(s.T, s.K)[toks]
    assert np.array_equal(part["qh"], full["qh"][rows])


def test_geometry_golden_matches_the_layer_shapes():
    g = {r[0]: int(r[1]) for r in _read_golden("geometry.txt")}
    for name in ("stream_all_1k", "chunk_8k", "long_32k", "skewed_4k"):
        s = S.shape(name)
        assert (s.H, s.K, s.E) == (g["hidden"], g["topk"], g["experts"])


def test_q2_0_code_one_is_zero_weight():
    """Under Q2_0, w = d * (q - 1): codes all 1 give zero weights, so the expert
    output is exactly zero; under the symmetric map the same codes give
    w = -d / 2, which is not."""
    s = S.custom(T=5, H=64, E=1, K=1, I=32)
    ex = S.expert(s, 0)
    ones = S.Expert(np.ones_like(ex.codes_gu), ex.scales_gu, np.ones_like(ex.codes_d), ex.scales_d)
    qx, sx = oracle.quantize(S.activations(s))
    h, qh, sh, D = oracle.expert_rows(ones, qx, sx, want_h=True, fmt="q2_0")
    assert np.all(h == 0) and np.all(qh == 0) and np.all(D == 0)
    h_sym, _, _, _ = oracle.expert_rows(ones, qx, sx, want_h=True, fmt="q2_sym")
    assert np.abs(h_sym).max() > 0
