"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: routing ids, grouping tables and the layer input's int8 codes and
scales bit-exact; routing weights within 1e-6 absolute (a softmax of the
fp32-class logits, whose accumulator chains are at most 8 blocks long:
measured 1.6e-7 to 8.4e-7); SwiGLU-output codes equal except at rounding
ties of the oracle's exact quotient (then off by one), at a rate below 1e-3;
the down stage fed the oracle's H codes within max|err| / max|ref| <= 1e-5
(and a per-output fp32 rounding bound); the layer output within
max|err| / max|ref| <= 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import packed_layout
import synthetic as S
from layers import (canonical_expert, check_h_codes, down_error_bound, gate_bound, getter, gpu_experts, rel_err,
                    shared_args)

pytestmark = pytest.mark.gpu

P_TOL = 1e-6     # routing weights: a softmax of the fp32-class logits
Y_TOL = 2e-3
DOWN_TOL = 1e-5   # the down stage alone, on the oracle's H codes
H_RATE = 1e-3     # largest share of SwiGLU-output codes that may sit one step off at a rounding tie


@pytest.fixture(scope="module")
def qm():
    import quantized_routed_expert_logits_amd as qm

    assert qm.strata_moe_device_supported(), "this test needs a gfx950 device"
    return qm


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ----------------------------------------------------------------- quantize
def test_quantize_bit_exact(qm):
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((700, 320)) * rng.choice([1e-6, 1e-2, 1.0, 300.0], (700, 1))).astype(np.float32)
    v[0, :32] = 0.0                                     # all-zero block
    v[1, :32] = np.float32(np.arange(32) - 15.5)        # half-way quotients with s == 1
    v[1, 0] = 127.0
    v[2, 32:64] = -2.75                                 # constant block
    v[3, :32] = np.float32(1e-40)                       # subnormal block
    q, s = qm.strata_moe_quantize(_t(v))
    qr, sr = oracle.quantize(v)
    assert np.array_equal(s.cpu().numpy(), sr)
    assert np.array_equal(q.cpu().numpy(), qr)


def test_quantize_full_size_input_bit_exact(qm):
    x = S.activations(S.shape("chunk_8k"))
    q, s = qm.strata_moe_quantize(_t(x))
    qr, sr = oracle.quantize(x)
    assert np.array_equal(s.cpu().numpy(), sr) and np.array_equal(q.cpu().numpy(), qr)


# --------------------------------------------------------------------- pack
@pytest.mark.parametrize("shape", [S.shape("tiny"), S.custom(T=1, H=384, E=3, K=1, I=192)])
def test_pack_unpack_round_trip(qm, shape):
    ex = gpu_experts(shape)
    cg, sg, cd, sd = qm.strata_moe_unpack(ex, 0, shape.E)
    for e in range(shape.E):
        c = canonical_expert(shape, e)
        assert np.array_equal(cg[e].cpu().numpy(), c.codes_gu)
        assert np.array_equal(sg[e].cpu().numpy().view(np.uint16), c.scales_gu)
        assert np.array_equal(cd[e].cpu().numpy(), c.codes_d)
        assert np.array_equal(sd[e].cpu().numpy().view(np.uint16), c.scales_d)


@pytest.mark.parametrize("shape", [S.shape("tiny"), S.custom(T=1, H=384, E=3, K=1, I=192),
                                   S.custom(T=1, H=2560, E=2, K=1, I=1024)])
def test_packed_layout_host_decode(qm, shape):
    """The packed blobs, copied to the host and decoded there from the layout's
    definition (tests/packed_layout.py), give back the canonical codes and
    scales: the packer writes the documented layout."""
    ex = gpu_experts(shape)
    gu = ex.gate_up.cpu().numpy()
    dn = ex.down.cpu().numpy()
    for e in range(shape.E):
        c = canonical_expert(shape, e)
        got = packed_layout.decode_expert(gu[e * ex.gate_up_stride:(e + 1) * ex.gate_up_stride],
                                          dn[e * ex.down_stride:(e + 1) * ex.down_stride], shape.H, shape.I)
        for g, want in zip(got, (c.codes_gu, c.scales_gu, c.codes_d, c.scales_d)):
            assert np.array_equal(g, want)


# -------------------------------------------------------------------- route
def _route_case(qm, x, wr, bias, K):
    ids, p = qm.strata_moe_route(_t(x), _t(wr), None if bias is None else _t(bias), K)
    ids_r, p_r = oracle.topk_softmax(oracle.router_logits(x, wr, bias), K)
    ids, p = ids.cpu().numpy(), p.cpu().numpy()
    assert np.array_equal(ids, ids_r)
    assert np.abs(p - p_r).max() <= P_TOL
    assert np.abs(p.astype(np.float64).sum(1) - 1).max() <= 1e-6


# the top-K takes a workgroup per token up to 1024 tokens, a wave per token above
@pytest.mark.parametrize("T", [200, 1500])
def test_route_many_experts(qm, T):
    """More than 512 experts: the selection keeps 16 logits per lane."""
    s = S.custom(T=T, H=256, E=1000, K=12, I=32)
    x, wr = S.activations(s, 6), S.router_weight(s, 6)
    wr[:, 777] = wr[:, 5]           # an exact tie across the two halves of the expert range
    _route_case(qm, x, wr, None, s.K)


@pytest.mark.parametrize("T", [100, 1100])
def test_route_every_expert_selected(qm, T):
    """K = E: every expert is selected, in rank order, and there is no rank
    K + 1 for the near-tie window to look at."""
    s = S.custom(T=T, H=256, E=12, K=12, I=32)
    x, wr = S.activations(s, 7), S.router_weight(s, 7)
    wr[:, 9] = wr[:, 2]  # an exact tie: lower index first
    _route_case(qm, x, wr, None, s.K)


def test_route_exact_ties_and_zero_router(qm):
    s = S.custom(T=300, H=512, E=40, K=7, I=32)
    x, wr = S.activations(s, 3), S.router_weight(s, 3)
    wr[:, 11] = wr[:, 4]            # exact ties: lower index first
    wr[:, 30] = wr[:, 29]
    _route_case(qm, x, wr, None, s.K)
    _route_case(qm, x, np.zeros_like(wr), None, s.K)   # all equal: 0..K-1, p = 1/K


@pytest.mark.parametrize("T", [512, 1536])
def test_route_near_ties_are_settled_exactly(qm, T):
    """Columns that differ by one fp32 ulp in a single entry: logits a few
    1e-7 apart, below fp32 accumulation noise."""
    s = S.custom(T=T, H=1024, E=64, K=10, I=32)
    x, wr = S.activations(s, 4), S.router_weight(s, 4)
    for a, b in [(3, 17), (40, 41), (9, 60)]:
        wr[:, b] = wr[:, a]
        wr[5, b] = np.nextafter(wr[5, a], np.float32(np.inf))
    _route_case(qm, x, wr, None, s.K)


def boundary_gaps(logits, K):
    """Per token, the exact logit gap between ranks K-1 and K (the smallest
    change that would alter the selected set)."""
    part = -np.partition(-logits, K, axis=1)[:, :K + 1]
    part = -np.sort(-part, axis=1)
    return part[:, K - 1] - part[:, K]


@pytest.mark.parametrize("name", ["tiny", "stream_all_1k", "chunk_8k", "long_32k", "skewed_4k"])
def test_route_all_tokens(qm, name):
    """Every token of the five workloads: ids bit-exact, p within P_TOL.
    Also reports the smallest exact boundary gap l_(K) - l_(K+1) over the
    tokens and how many tokens sit below 1e-6 (the margin the near-tie
    re-score has to settle)."""
    s = S.shape(name)
    x, wr, bias = S.activations(s), S.router_weight(s), S.router_bias(s)
    ids, p = qm.strata_moe_route(_t(x), _t(wr), None if bias is None else _t(bias), s.K)
    logits = oracle.router_logits(x, wr, bias)
    ids_r, p_r = oracle.topk_softmax(logits, s.K)
    gap = boundary_gaps(logits, s.K)
    ids, p = ids.cpu().numpy(), p.cpu().numpy()
    print(f"{name}: {s.T} tokens, min boundary gap {gap.min():.3e}, tokens below 1e-6: {(gap < 1e-6).sum()}, "
          f"mismatched tokens: {int((ids != ids_r).any(1).sum())}, max |dp| {np.abs(p - p_r).max():.2e}, "
          f"tokens with |dp| > 1e-6: {int((np.abs(p - p_r) > 1e-6).any(1).sum())}")
    assert np.array_equal(ids, ids_r)
    assert np.abs(p - p_r).max() <= P_TOL
    assert np.abs(p.astype(np.float64).sum(1) - 1).max() <= 1e-6


def router_error_bound(x, wr, bias=None):
    """Per-token bound of the GPU logits' error, as the routing kernels model
    it: three fp16 products per term (hi and lo halves, 2^-20 of |x||w|
    together), each passing through at most 31 additions inside an MFMA and
    3 H / 32 accumulator additions, plus a few for the split reduction and the
    bias, each within 2^-23 of its result; sum_h |x_h w_he| <=
    ||x||_2 ||w_e||_2.  The bias passes through at most 9 roundings (8 split
    ranges and its own addition).  This counts one accumulator chain over all
    of H, wider than the kernels' own bound (their chains end every 8 k blocks
    into fp64 sums)."""
    H = x.shape[1]
    c = (3 * H / 32 + 40) * 2.0 ** -23 + 2.0 ** -20
    xn = np.linalg.norm(x.astype(np.float64), axis=1)
    wn = np.linalg.norm(wr.astype(np.float64), axis=0).max()
    bm = 0.0 if bias is None else float(np.abs(bias.astype(np.float64)).max())
    return c * xn * wn + 9 * 2.0 ** -23 * bm


def test_route_outlier_channels(qm):
    """Heavy-tailed inputs with a few outlier channels (Student-t values, 8
    channels scaled by 200): logits far above the synthetic scale, where a
    window fixed by the logits' size alone would be too narrow.  Every token's
    ids bit-exact; p within the softmax's response to the logit error bound."""
    s = S.custom(T=2048, H=2560, E=512, K=10, I=32)
    rng = np.random.default_rng(21)
    x = rng.standard_t(3, (s.T, s.H))
    x[:, rng.choice(s.H, 8, replace=False)] *= 200.0
    x = x.astype(np.float32)
    wr = S.router_weight(s, 21)
    wr[:, 300] = wr[:, 299]            # an exact tie
    wr[:, 301] = wr[:, 299]
    wr[7, 301] = np.nextafter(wr[7, 299], np.float32(np.inf))  # and a one-ulp near tie
    ids, p = qm.strata_moe_route(_t(x), _t(wr), None, s.K)
    logits = oracle.router_logits(x, wr)
    ids_r, p_r = oracle.topk_softmax(logits, s.K)
    ids, p = ids.cpu().numpy(), p.cpu().numpy()
    print(f"outlier channels: logits up to {np.abs(logits).max():.1f}, min boundary gap "
          f"{boundary_gaps(logits, s.K).min():.3e}, mismatched tokens {int((ids != ids_r).any(1).sum())}")
    assert np.array_equal(ids, ids_r)
    tol = 2.0 * router_error_bound(x, wr)[:, None] + 1e-6
    assert np.all(np.abs(p - p_r) <= tol)


@pytest.mark.parametrize("T", [300, 1500])
def test_route_large_bias(qm, T):
    """A bias of 1e5 on every expert: there the fp32 logits are 7.8e-3 apart,
    and each of the router's split ranges rounds the running sum near 1e5, so
    two experts whose exact logits are less than about two such steps apart
    can come out one step apart in the wrong order.  Columns 20..40 form a
    ladder (w_e = w_20 + (e - 20) c u) whose logits are a fraction of a step
    apart for a typical token, and carry 10 more bias, so the top K come from
    the ladder.  The dot products' own error is about 2e-4 here: only the
    bias's share of the error bound puts such pairs inside the near-tie window
    (a host model of the split sums misranks 5 of 300 and 14 of 1500 tokens
    outside a window without it).  ids bit-exact; p within the softmax's
    response to the bound."""
    s = S.custom(T=T, H=256, E=64, K=4, I=32)
    x, wr = S.activations(s, 8), S.router_weight(s, 8)
    u = np.random.default_rng(9).standard_normal(s.H)
    for e in range(21, 41):
        wr[:, e] = (wr[:, 20].astype(np.float64) + (e - 20) * 4e-4 * u).astype(np.float32)
    bias = np.full(s.E, 1e5, np.float32)
    bias[20:41] = np.float32(1e5 + 10)
    ids, p = qm.strata_moe_route(_t(x), _t(wr), _t(bias), s.K)
    logits = oracle.router_logits(x, wr, bias)
    ids_r, p_r = oracle.topk_softmax(logits, s.K)
    ids, p = ids.cpu().numpy(), p.cpu().numpy()
    print(f"large bias: min boundary gap {boundary_gaps(logits, s.K).min():.3e}, "
          f"mismatched tokens {int((ids != ids_r).any(1).sum())}")
    assert np.array_equal(ids, ids_r)
    tol = 2.0 * router_error_bound(x, wr, bias)[:, None] + 1e-6
    assert np.all(np.abs(p - p_r) <= tol)


# -------------------------------------------------------------------- group
# n = T K pairs: up to one chunk of 2048 takes the one-workgroup kernel (204 x 10 is the last such), more
# the three-kernel path
@pytest.mark.parametrize("T,E,K,skew", [(64, 16, 2, 0.0), (3000, 512, 10, 0.0), (4096, 512, 10, 3.0),
                                        (32768, 512, 10, 0.0), (257, 1024, 16, 0.0), (9, 1, 1, 0.0),
                                        (204, 512, 10, 0.0), (205, 512, 10, 0.0), (128, 1024, 16, 3.0),
                                        (1024, 512, 10, 3.0)])
def test_group_bit_exact(qm, T, E, K, skew):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)) - skew * np.log1p(np.arange(E))[None, :]
    ids, _ = oracle.topk_softmax(logits, K)
    offsets, src, slot = qm.strata_moe_group(_t(ids), E)
    o_r, s_r, sl_r = oracle.group(ids, E)
    assert np.array_equal(offsets.cpu().numpy(), o_r)
    assert np.array_equal(src.cpu().numpy(), s_r)
    assert np.array_equal(slot.cpu().numpy(), sl_r)


def test_group_rejects_out_of_range_ids(qm):
    ids = np.zeros((100, 4), np.int32)
    ids[:, 1], ids[:, 2], ids[:, 3] = 1, 2, 3
    ids[57, 2] = 16
    with pytest.raises(qm.StrataMoeError) as ei:
        qm.strata_moe_group(_t(ids), 16)
    assert ei.value.code == qm.EDATA


# ------------------------------------------------------------ expert stages
def _stage_ref(s):
    x, wr = S.activations(s), S.router_weight(s)
    return x, wr, oracle.layer(x, wr, S.router_bias(s), getter(s), s.E, s.K, want_h=True, fmt=s.fmt)


STAGE_SHAPES = [S.shape("tiny"), S.custom(T=300, H=256, E=12, K=3, I=128), S.custom(T=70, H=640, E=5, K=2, I=192),
                S.custom(T=2000, H=384, E=3, K=2, I=64),
                # the pages' Q2_0 map, and its FFN width 640 (20 blocks: not a multiple of 8)
                S.custom(T=300, H=256, E=12, K=3, I=128, fmt="q2_0"), S.custom(T=160, H=512, E=6, K=2, I=640, fmt="q2_0"),
                # about 40 rows per expert: 3-tile chunks in the small-chunk kernel
                S.custom(T=200, H=256, E=10, K=2, I=128),
                # the production widths H = 2560, I = 1024 at small T: three 32-block chunks
                # of the offset pass, the 8-deep record ring; about 24 rows per expert (the
                # small-chunk kernel) and about 107 (the 4-wave kernel, 7 tiles)
                S.custom(T=48, H=2560, E=4, K=2, I=1024), S.custom(T=160, H=2560, E=3, K=2, I=1024),
                S.custom(T=96, H=2560, E=4, K=2, I=640, fmt="q2_0"),
                # one or two rows per expert: the GEMV kernel (decode-window sizes)
                S.custom(T=20, H=256, E=64, K=4, I=128), S.custom(T=24, H=512, E=48, K=3, I=640, fmt="q2_0"),
                S.custom(T=16, H=2560, E=32, K=2, I=1024)]


@pytest.mark.parametrize("s", STAGE_SHAPES, ids=lambda s: s.name)
def test_gate_up_stage(qm, s):
    x, wr, ref = _stage_ref(s)
    ex = gpu_experts(s)
    qh, sh = qm.strata_moe_gate_up(_t(ref["qx"]), _t(ref["sx"]), _t(ref["offsets"]), _t(ref["src"]), s.K, ex)
    rate = check_h_codes(qh.cpu().numpy(), sh.cpu().numpy(), ref["h"], ref["qh"], ref["sh"])
    print(f"{s.name}: H-code mismatch rate {rate:.2e}")
    assert rate < H_RATE


@pytest.mark.parametrize("s", STAGE_SHAPES, ids=lambda s: s.name)
def test_down_stage(qm, s):
    x, wr, ref = _stage_ref(s)
    ex = gpu_experts(s)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    qm.strata_moe_down(_t(ref["qh"]), _t(ref["sh"]), _t(ref["offsets"]), _t(ref["src"]), _t(ref["slot"]),
                       _t(ref["p"].astype(np.float32)), ex, out)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref["y"])
    bound = down_error_bound(s, ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3f}"
    rel = rel_err(out.cpu().numpy(), ref["y"])
    print(f"{s.name}: down stage max|dy|/max|y| = {rel:.2e}")
    assert rel <= DOWN_TOL


# --------------------------------------------------------------- the layer
LAYER_SHAPES = STAGE_SHAPES + [S.custom(T=129, H=256, E=8, K=4, I=64, skewed=True),
                               # the largest widths the library takes (H = I = 4096), and the most
                               # experts and pairs per token (E = 1024, K = 16)
                               S.custom(T=24, H=4096, E=4, K=2, I=4096), S.custom(T=64, H=256, E=1024, K=16, I=64),
                               # every token on every expert (K = E: no rank K + 1 to compare against)
                               S.custom(T=100, H=256, E=6, K=6, I=64),
                               # a single token (one row for each of K experts)
                               S.custom(T=1, H=256, E=16, K=4, I=128)]


@pytest.mark.parametrize("s", LAYER_SHAPES, ids=lambda s: s.name)
def test_layer_all_intermediates(qm, s):
    x, wr, ref = _stage_ref(s)
    ex = gpu_experts(s)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    d = qm.strata_moe_prefill_debug(_t(x), _t(wr), ex, s.K, out)
    g = {k: v.cpu().numpy() for k, v in d.items()}
    for k in ("ids", "offsets", "src", "slot", "qx", "sx"):
        assert np.array_equal(g[k], ref[k]), k
    assert np.abs(g["p"] - ref["p"]).max() <= P_TOL
    assert check_h_codes(g["qh"], g["sh"], ref["h"], ref["qh"], ref["sh"]) < H_RATE
    assert rel_err(g["out"], ref["y"]) <= Y_TOL


@pytest.mark.parametrize("s", LAYER_SHAPES, ids=lambda s: s.name)
def test_layer_down_operand_from_epilogue_matches_stage_path(qm, s):
    # In the layer the gate/up epilogue writes the down GEMM's tiled fp16
    # operand and block values of the offset pass itself; the single-step
    # down entry builds both from the int8 H codes.  Same bits either way,
    # and the plain entry (which writes no int8 H codes) matches the debug
    # entry (which does).
    x, wr = S.activations(s), S.router_weight(s)
    ex = gpu_experts(s)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    d = qm.strata_moe_prefill_debug(_t(x), _t(wr), ex, s.K, out)
    y = qm.strata_moe_down(d["qh"], d["sh"], d["offsets"], d["src"], d["slot"], d["p"], ex, torch.empty_like(out))
    assert torch.equal(y, out)
    y2 = qm.strata_moe_prefill(_t(x), _t(wr), ex, s.K, torch.empty_like(out))
    assert torch.equal(y2, out)


def test_layer_every_token_on_the_same_experts(qm):
    # A router bias sends every token to the same K experts: each of them
    # gets all T rows (six chunks of the 4-wave kernels apiece), the other
    # experts none.
    s = S.custom(T=1000, H=256, E=24, K=4, I=128)
    x, wr = S.activations(s), S.router_weight(s)
    bias = np.zeros(s.E, np.float32)
    hot = [3, 7, 11, 20]
    bias[hot] = 100.0
    ref = oracle.layer(x, wr, bias, getter(s), s.E, s.K, want_h=True, fmt=s.fmt)
    ex = gpu_experts(s).with_router_bias(_t(bias))
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    d = qm.strata_moe_prefill_debug(_t(x), _t(wr), ex, s.K, out)
    g = {k: v.cpu().numpy() for k, v in d.items()}
    assert np.array_equal(np.sort(g["ids"], axis=1), np.tile(hot, (s.T, 1)))
    counts = np.diff(g["offsets"])
    assert np.array_equal(np.nonzero(counts)[0], hot) and np.all(counts[hot] == s.T)
    for k in ("ids", "offsets", "src", "slot", "qx", "sx"):
        assert np.array_equal(g[k], ref[k]), k
    # logits near 100 are 7.6e-6 apart in fp32: p within the softmax's response to the logits' bound
    tol = 2.0 * router_error_bound(x, wr, bias)[:, None] + 1e-6
    assert np.all(np.abs(g["p"] - ref["p"]) <= tol)
    assert check_h_codes(g["qh"], g["sh"], ref["h"], ref["qh"], ref["sh"]) < H_RATE
    assert rel_err(g["out"], ref["y"]) <= Y_TOL
    y = qm.strata_moe_prefill(_t(x), _t(wr), ex, s.K, torch.empty_like(out))
    assert torch.equal(y, out)


SHARED_SHAPES = [S.custom(T=200, H=256, E=10, K=3, I=128, shared=True),
                 S.custom(T=160, H=512, E=6, K=2, I=640, fmt="q2_0", shared=True),
                 S.custom(T=129, H=256, E=8, K=4, I=64, skewed=True, shared=True),
                 # with the shared expert the grouping reaches E + 1 = 1024 experts and K + 1 = 16 slots
                 S.custom(T=64, H=256, E=1023, K=15, I=64, shared=True)]


@pytest.mark.parametrize("s", SHARED_SHAPES, ids=lambda s: s.name)
def test_layer_with_shared_expert(qm, s):
    # the shared expert is pair slot K of every token (expert E, weight its
    # gate); the routed part keeps the routed-only grouping order
    x, wr = S.activations(s), S.router_weight(s)
    ref = oracle.layer(x, wr, S.router_bias(s), getter(s), s.E, s.K, want_h=True, fmt=s.fmt, shared=shared_args(s))
    ex = gpu_experts(s)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    d = qm.strata_moe_prefill_debug(_t(x), _t(wr), ex, s.K, out)
    g = {k: v.cpu().numpy() for k, v in d.items()}
    T, K, E = s.T, s.K, s.E
    assert np.array_equal(g["ids"][:, :K], ref["ids"]) and np.all(g["ids"][:, K] == E)
    assert np.abs(g["p"][:, :K] - ref["p"]).max() <= P_TOL
    assert np.all(np.abs(g["p"][:, K] - ref["shared"]["g"]) <= gate_bound(x, S.shared_gate_weight(s)))
    _check_grouping_props(g, T, K + 1, E + 1)
    o0 = int(g["offsets"][E])
    assert np.array_equal(g["offsets"][:E + 1], ref["offsets"]) and np.array_equal(g["src"][:o0], ref["src"])
    assert np.array_equal(g["src"][o0:], np.arange(T))  # the shared expert's rows: every token in order
    for k in ("qx", "sx"):
        assert np.array_equal(g[k], ref[k]), k
    assert check_h_codes(g["qh"][:o0], g["sh"][:o0], ref["h"], ref["qh"], ref["sh"]) < H_RATE
    rs = ref["shared"]
    assert check_h_codes(g["qh"][o0:], g["sh"][o0:], rs["h"], rs["qh"], rs["sh"]) < H_RATE
    assert rel_err(g["out"], ref["y"]) <= Y_TOL
    # the plain entry point gives the same bits
    y = qm.strata_moe_prefill(_t(x), _t(wr), ex, s.K, torch.empty_like(out))
    assert torch.equal(y, out)


def test_layer_zero_input_and_repeat(qm):
    s = S.shape("tiny")
    ex = gpu_experts(s)
    wr = _t(S.router_weight(s))
    out = torch.full((s.T, s.H), 7.0, device="cuda")
    qm.strata_moe_prefill(torch.zeros((s.T, s.H), device="cuda"), wr, ex, s.K, out)
    assert torch.count_nonzero(out).item() == 0
    x = _t(S.activations(s))
    a = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x)).clone()
    b = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x))
    assert torch.equal(a, b)  # the combine adds each token's rows in a fixed order


@pytest.mark.parametrize("s", [S.shape("tiny"), S.custom(T=300, H=256, E=12, K=3, I=128),
                               S.custom(T=129, H=256, E=8, K=4, I=64, skewed=True)], ids=lambda s: s.name)
def test_layer_prepared_router_is_identical(qm, s):
    # the router matrix prepared once (strata_moe_prepare_router) gives the
    # same bits as preparing it in every call; a later call with the other
    # form in between checks that neither leaves state behind
    ex = gpu_experts(s)
    wr = _t(S.router_weight(s))
    x = _t(S.activations(s))
    exp = ex.with_prepared_router(wr)
    a = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x)).clone()
    b = qm.strata_moe_prefill(x, wr, exp, s.K, torch.empty_like(x)).clone()
    c = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x))
    assert torch.equal(a, b) and torch.equal(a, c)


def test_layer_zero_tokens(qm):
    s = S.shape("tiny")
    ex = gpu_experts(s)
    x = torch.empty((0, s.H), device="cuda")
    qm.strata_moe_prefill(x, _t(S.router_weight(s)), ex, s.K, torch.empty_like(x))


# ------------------------------------------------------- small-T kernels
SMALL_T = [S.shape("window_32"), S.custom(T=20, H=256, E=64, K=4, I=128),
           S.custom(T=24, H=512, E=48, K=3, I=640, fmt="q2_0"),
           S.custom(T=64, H=256, E=32, K=3, I=192),  # 6 rows per expert: the GEMV only when forced
           # T <= 8: every chunk is the GEMV's (the MFMA kernels and the tiled H are not launched)
           S.custom(T=8, H=256, E=16, K=4, I=128), S.custom(T=6, H=512, E=12, K=3, I=192, fmt="q2_0")]


@pytest.mark.parametrize("s", SMALL_T, ids=lambda s: s.name)
def test_small_t_kernel_choices(qm, s):
    """The layer at decode-window sizes through its kernel choices for short
    chunks: the default (the int8 GEMV on chunks of <= 8 rows where the
    experts average <= 2 rows, two rows per pass), the MFMA kernels only
    (FLAG_NO_GEMV), the GEMV on per-slot q8_1 inputs (FLAG_PER_SLOT_Q8) and
    the GEMV at any average (FLAG_GEMV_ALWAYS, alone and with the per-slot
    arm); each against the oracle."""
    x, wr, ref = _stage_ref(s)
    ex = gpu_experts(s)
    sizes = np.diff(ref["offsets"])
    assert np.count_nonzero((sizes > 0) & (sizes <= 2)) > 0  # single-pass chunks
    assert np.count_nonzero((sizes > 2) & (sizes <= 8)) > 0  # several passes
    print(f"{s.name}: rows per expert {s.T * s.K / s.E:.2f} on average, chunk sizes up to {sizes.max()}")
    outs = {}
    for flags in (0, qm.FLAG_NO_GEMV, qm.FLAG_PER_SLOT_Q8, qm.FLAG_GEMV_ALWAYS,
                  qm.FLAG_GEMV_ALWAYS | qm.FLAG_PER_SLOT_Q8):
        out = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
        d = qm.strata_moe_prefill_debug(_t(x), _t(wr), ex.with_flags(flags), s.K, out)
        g = {k: v.cpu().numpy() for k, v in d.items()}
        for k in ("ids", "offsets", "src", "slot", "qx", "sx"):
            assert np.array_equal(g[k], ref[k]), (flags, k)
        rate = check_h_codes(g["qh"], g["sh"], ref["h"], ref["qh"], ref["sh"])
        err = rel_err(g["out"], ref["y"])
        print(f"{s.name} flags {flags}: max|dy|/max|y| = {err:.2e}, H-code mismatch rate {rate:.2e}")
        assert rate < H_RATE and err <= Y_TOL
        outs[flags] = g["out"]
    # the arms are not compared with each other bit for bit: their fp32 rounding orders differ, so an
    # H code at a rounding near-tie may go either way (each is checked against the oracle above)


# ------------------------------------------------- full-size layers, sampled
def _check_grouping_props(g, T, K, E):
    offsets, src, slot, ids = g["offsets"], g["src"], g["slot"], g["ids"].reshape(-1)
    n = T * K
    assert offsets[0] == 0 and offsets[E] == n and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.diff(offsets), np.bincount(ids, minlength=E))
    assert np.array_equal(np.bincount(src, minlength=T), np.full(T, K))
    assert np.array_equal(np.sort(slot), np.arange(n))
    assert np.array_equal(src[slot], np.arange(n) // K)
    grp = np.repeat(np.arange(E), np.diff(offsets))
    assert np.array_equal(grp[slot], ids)
    inner = np.diff(src)[np.diff(grp) == 0]
    assert np.all(inner > 0)  # ascending tokens within each expert


@pytest.mark.parametrize("name", ["stream_all_1k", "chunk_8k", "skewed_4k", "long_32k", "pages_q2_0_2k",
                                  "chunk_8k_shared", "pages_shared_2k", "short_256", "window_32"])
def test_full_layer_sampled(qm, name):
    _full_layer_sampled(qm, S.shape(name), name)


def test_full_layer_longest_call(qm):
    """The longest call the library takes at these widths: its tiled operands
    ((T K + 15 E) x 2560 fp16 values) stay under 2 GiB up to 41,175 tokens.
    At 40,960 they hold 2.14e9 bytes, so every buffer size and byte offset of
    the GEMMs' buffer resources sits just under 2^31."""
    s = S.custom(T=40960, H=2560, E=512, K=10, I=1024)
    _full_layer_sampled(qm, s, "longest call")


def _full_layer_sampled(qm, s, name):
    ex = gpu_experts(s)
    x, wr, bias = S.activations(s), S.router_weight(s), S.router_bias(s)
    xt, wt = _t(x), _t(wr)
    out = torch.empty_like(xt)
    qm.strata_moe_prefill(xt, wt, ex, s.K, out)          # the launch the benchmark times
    y = out.cpu().numpy()
    d = qm.strata_moe_prefill_debug(xt, wt, ex, s.K, torch.empty_like(xt))
    g = {k: v.cpu().numpy() for k, v in d.items() if k in ("ids", "p", "offsets", "src", "slot", "qx", "sx", "qh", "sh")}
    _check_grouping_props(g, s.T, s.K + s.shared, s.E + s.shared)
    rng = np.random.default_rng(5)
    tok = [0, s.T - 1] + list(rng.choice(s.T, 30, replace=False))
    if s.skewed:  # tokens of the busiest expert (its tiles run last in their group)
        busiest = int(np.argmax(np.diff(g["offsets"])))
        rows = g["src"][g["offsets"][busiest]:g["offsets"][busiest + 1]]
        tok += list(rows[-8:])
    tok = np.unique(tok)
    ref = oracle.layer_tokens(x, wr, bias, getter(s), s.K, tok, fmt=s.fmt, shared=shared_args(s))
    assert np.array_equal(g["ids"][tok][:, :s.K], ref["ids"])
    assert np.abs(g["p"][tok][:, :s.K] - ref["p"]).max() <= P_TOL
    assert np.array_equal(g["qx"][tok], ref["qx"]) and np.array_equal(g["sx"][tok], ref["sx"])
    # the sampled tokens' routed rows: pair t*Kg + k sits in grouped row slot[t*Kg + k]
    Kg = s.K + s.shared
    rows = g["slot"].reshape(s.T, Kg)[tok][:, :s.K].reshape(-1)
    I = s.I
    rate = check_h_codes(g["qh"][rows], g["sh"][rows], ref["h"].reshape(-1, I), ref["qh"].reshape(-1, I),
                         ref["sh"].reshape(-1, I // 32))
    err = rel_err(y[tok], ref["y"])
    print(f"{name}: {len(tok)} sampled tokens, max|dy|/max|y| = {err:.2e}, H-code mismatch rate {rate:.2e}")
    assert rate < H_RATE
    assert err <= Y_TOL
