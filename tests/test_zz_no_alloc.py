"""strata_moe_prefill_noalloc (the layer on the library's fixed scratch array,
for callers that cannot allocate) against strata_moe_prefill: the same
launches on the same data, so the same bits; two calls in a row, the second
smaller, at test sizes and at the 1024-token production chunk; and a call too
large for the array rejected before anything runs."""
import numpy as np
import pytest
import torch

import synthetic as S
from layers import gpu_experts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qm():
    import quantized_routed_expert_logits_amd as qm

    assert qm.strata_moe_device_supported(), "this test needs a gfx950 device"
    return qm


def _inputs(s):
    return torch.from_numpy(S.activations(s)).cuda(), torch.from_numpy(S.router_weight(s)).cuda()


@pytest.mark.parametrize("big,small", [
    (S.custom(T=300, H=256, E=12, K=3, I=128), S.custom(T=77, H=256, E=12, K=3, I=128)),
    (S.custom(T=160, H=512, E=6, K=2, I=640, fmt="q2_0", shared=True),
     S.custom(T=33, H=512, E=6, K=2, I=640, fmt="q2_0", shared=True)),
    (S.shape("stream_all_1k"), S.shape("short_256")),
    # the second call takes the GEMV (0.6 rows per expert) after an MFMA-only call
    (S.shape("short_256"), S.shape("window_32")),
], ids=lambda s: s.name)
def test_noalloc_matches_prefill_on_two_calls(qm, big, small):
    ex = gpu_experts(big)
    assert (small.E, small.H, small.I, small.fmt, small.shared) == (big.E, big.H, big.I, big.fmt, big.shared)
    for s in (big, small):  # the second call is smaller and reuses the same scratch
        x, wr = _inputs(s)
        y = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x))
        out = torch.full_like(x, float("nan"))
        lib = qm.library()
        import ctypes

        rc = lib.strata_moe_prefill_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(wr.data_ptr()),
                                            ctypes.byref(ex.struct), s.T, s.K, ctypes.c_void_p(out.data_ptr()),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, qm.strata_moe_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, y), s.name


def test_noalloc_rejects_a_call_larger_than_its_scratch(qm):
    s = S.shape("stream_all_1k")
    ex = gpu_experts(s)
    T = 4096  # about 880 MiB of workspace at this layer's sizes
    assert qm.strata_moe_workspace_bytes(T, s.K, ex) > qm.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, s.H), device="cuda")
    wr = torch.from_numpy(S.router_weight(s)).cuda()
    out = torch.full_like(x, 7.0)
    with pytest.raises(qm.StrataMoeError) as ei:
        qm.strata_moe_prefill_noalloc(x, wr, ex, s.K, out)
    assert ei.value.code == qm.EINVAL and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing ran


def test_noalloc_at_its_largest_call(qm):
    """The longest call whose workspace fits the array (about 2,250 tokens at
    H = 2560, I = 1024, E = 512, K = 10) against strata_moe_prefill, bit for
    bit; one token more is rejected."""
    base = S.shape("stream_all_1k")
    ex = gpu_experts(base)
    lo, hi = 1, 1 << 16  # the largest T whose workspace fits, by bisection on the sizing call
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if qm.strata_moe_workspace_bytes(mid, base.K, ex) <= qm.NOALLOC_SCRATCH_BYTES else (lo, mid - 1)
    s = S.custom(T=lo, H=base.H, E=base.E, K=base.K, I=base.I)
    x, wr = _inputs(s)
    y = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x))
    out = torch.full_like(x, float("nan"))
    qm.strata_moe_prefill_noalloc(x, wr, ex, s.K, out)
    torch.cuda.synchronize()
    assert torch.equal(out, y), s.T
    x1 = torch.zeros((lo + 1, s.H), device="cuda")
    with pytest.raises(qm.StrataMoeError) as ei:
        qm.strata_moe_prefill_noalloc(x1, wr, ex, s.K, torch.empty_like(x1))
    assert ei.value.code == qm.EINVAL


@pytest.mark.parametrize("s", [S.custom(T=300, H=256, E=12, K=3, I=128), S.shape("window_32")], ids=lambda s: s.name)
def test_noalloc_call_captured_in_a_graph(qm, s):
    # The entry point makes no allocation, memset or synchronisation, so a
    # caller can capture it in a HIP graph.  Each replay, with the program's
    # own eager work and synchronisations between replays, gives the bits of
    # the eager call.
    ex = gpu_experts(s)
    x, wr = _inputs(s)
    ref = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x))
    torch.cuda.synchronize()
    out = torch.empty_like(x)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # one eager call first on the capture stream
        qm.strata_moe_prefill_noalloc(x, wr, ex, s.K, out, stream=stream)
    stream.synchronize()
    assert torch.equal(out, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qm.strata_moe_prefill_noalloc(x, wr, ex, s.K, out, stream=stream)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        y = qm.strata_moe_prefill(x, wr, ex, s.K, torch.empty_like(x))  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
