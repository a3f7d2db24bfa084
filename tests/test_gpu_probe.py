"""The matrix unit's behaviour that the routing kernels' error bound rests on:
v_mfma_f32_16x16x32_f16 forms its fp16 products exactly, sums the 32 of them
before it adds the accumulator (so the accumulator sees one addition per
instruction), and that sum is within 31 fp32 additions' error (2^-23 each,
truncation included) of the exact one.  Crafted operands make a wrong premise
visible: an accumulator added first would lose the small products, and a sum
outside the bound would show on the cancelling cases.

The probe's rates must also stay below the published dense peaks: a rate
above its peak means the compiler dropped work from the measured kernel."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

U2 = 2.0 ** -23  # one fp32 addition's error, rounding or truncation


@pytest.fixture(scope="module")
def probe():
    from quantized_routed_expert_logits_amd import probe
    return probe


def _case(probe, prods, c0=0.0):
    """Output (0, 0) of one MFMA whose row 0 / column 0 products are prods
    (pairs (a, b), exact in fp16) and whose accumulator entry is c0."""
    A = np.zeros((16, 32), np.float32)
    B = np.zeros((32, 16), np.float32)
    C = np.zeros((16, 16), np.float32)
    for k, (a, b) in enumerate(prods):
        A[0, k], B[k, 0] = a, b
    C[0, 0] = c0
    return float(probe.strata_probe_mfma_f16(A, B, C)[0, 0])


def _within_model(probe, prods, c0=0.0):
    d = _case(probe, prods, c0)
    p = [float(np.float16(a)) * float(np.float16(b)) for a, b in prods]
    exact_sum = float(np.sum(np.array(p, np.float64)))
    # the products' sum within 31 additions' error, then one addition of c0
    bound = 31 * U2 * float(np.abs(p).sum()) + U2 * (abs(exact_sum) + abs(c0)) * 1.01
    return abs(d - (exact_sum + c0)) <= bound, d


def test_mfma_f16_products_are_exact(probe):
    # fp16 x fp16 needs at most 22 significant bits: (1 + 2^-10)^2 = 1 + 2^-9 + 2^-20
    v = 1.0 + 2.0 ** -10
    assert _case(probe, [(v, v)]) == v * v


def test_mfma_f16_adds_the_accumulator_once(probe):
    # 32 products of 1/2 onto 2^24: one at a time each would round away (ulp 2); summed first they give 16
    assert _case(probe, [(1.0, 0.5)] * 32, 2.0 ** 24) == 2.0 ** 24 + 16


def test_mfma_f16_sum_within_the_error_model(probe):
    cases = [
        [(2.0 ** 10, 2.0 ** 10), (2.0 ** -10, 2.0 ** -10), (-(2.0 ** 10), 2.0 ** 10)],  # cancellation
        [(2.0 ** 10, 2.0 ** 10)] + [(1.0, 2.0 ** -5)] * 31,                             # big first
        [(1.0, 2.0 ** -5)] * 31 + [(2.0 ** 10, 2.0 ** 10)],                             # big last
        [(1.0, 1.0), (3.0 * 2.0 ** -13, 2.0 ** -12)],                                   # 0.75 ulp below 1
    ]
    rng = np.random.default_rng(3)
    for _ in range(20):  # random mixed signs and magnitudes (normal fp16 values)
        a = rng.choice([-1.0, 1.0], 32) * (0.5 + rng.random(32)) * 2.0 ** rng.integers(-8, 8, 32)
        b = rng.choice([-1.0, 1.0], 32) * (0.5 + rng.random(32)) * 2.0 ** rng.integers(-8, 8, 32)
        cases.append(list(zip(np.float16(a).astype(float), np.float16(b).astype(float))))
    for prods in cases:
        ok, d = _within_model(probe, prods)
        assert ok, (prods[:3], d)
    ok, d = _within_model(probe, [(1.0, 0.5)] * 32, 2.0 ** 24)
    assert ok


# published dense peaks of the MI355X matrix unit (no sparsity), ops/s
PEAK_F16 = 2.5e15
PEAK_I8 = 5.0e15


def test_probe_rates_below_published_peaks(probe):
    for kind in probe.KINDS:
        rate, _ = probe.strata_probe_mfma_rate(kind)
        peak = PEAK_F16 if kind.startswith("f16") else PEAK_I8
        assert 0 < rate <= 1.05 * peak, (kind, rate)
    # a scaled output-block is 32 multiply-adds (64 ops) on the fp16 or int8 unit
    for i8 in (False, True):
        rate, _ = probe.strata_probe_scaled_blocks(i8)
        assert 0 < rate * 64 <= 1.05 * (PEAK_I8 if i8 else PEAK_F16), (i8, rate)
    for form in ("16x16x32", "32x32x16"):
        for tiles in (1, 6):
            rate, _ = probe.strata_probe_scaled_tiles(form, tiles)
            print(f"scaled tiles {form} x {tiles}: {rate / 1e12:.1f} T output-blocks/s")
            assert 0 < rate * 64 <= 1.05 * PEAK_F16, (form, tiles, rate)
    for step in (0, 1, 2):
        rate, _ = probe.strata_probe_block_step(step)
        print(f"block step {step}: {rate / 1e12:.1f} T output-blocks/s")
        assert 0 < rate * 64 <= 1.05 * PEAK_F16, (step, rate)
