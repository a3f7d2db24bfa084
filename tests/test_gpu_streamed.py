"""The streamed layer (every expert DMA'd from pinned host memory through a
ring of device slots while the layer runs) against the resident layer: the
same kernels over the same chunks, so the outputs must be the same bits, for
rings smaller than one batch of experts up to rings larger than the layer,
over consecutive calls that wrap around the ring."""
import numpy as np
import pytest
import torch

import synthetic as S
from layers import canonical_expert, gpu_experts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qm():
    import quantized_routed_expert_logits_amd as qm

    assert qm.strata_moe_device_supported(), "this test needs a gfx950 device"
    return qm


def _host_experts(qm, s, seed=0, chunk=32):
    ex = qm.HostExperts(s.E, s.H, s.I, fmt=s.fmt, shared=s.shared)
    nb = s.E + s.shared
    for e0 in range(0, nb, chunk):
        parts = [canonical_expert(s, e, seed) for e in range(e0, min(nb, e0 + chunk))]
        ex.pack(e0, np.stack([p.codes_gu for p in parts]), np.stack([p.scales_gu for p in parts]),
                np.stack([p.codes_d for p in parts]), np.stack([p.scales_d for p in parts]))
    if s.shared:
        ex = ex.with_shared_gate(torch.from_numpy(S.shared_gate_weight(s, seed)).cuda())
    bias = S.router_bias(s, seed)
    return ex.with_router_bias(None if bias is None else torch.from_numpy(bias).cuda())


CASES = [(S.shape("tiny"), 3), (S.shape("tiny"), 7), (S.shape("tiny"), 64),
         (S.custom(T=300, H=256, E=12, K=3, I=128), 4),
         (S.custom(T=129, H=256, E=8, K=4, I=64, skewed=True), 1),
         (S.custom(T=160, H=512, E=6, K=2, I=640, fmt="q2_0", shared=True), 5),
         (S.custom(T=200, H=256, E=10, K=3, I=128, shared=True), 2),
         (S.custom(T=20, H=256, E=64, K=4, I=128), 5)]  # one or two rows per expert: the GEMV


@pytest.mark.parametrize("s,R", CASES, ids=lambda v: v.name if hasattr(v, "name") else f"R{v}")
def test_streamed_layer_is_bitwise_the_resident_layer(qm, s, R):
    x = torch.from_numpy(S.activations(s)).cuda()
    wr = torch.from_numpy(S.router_weight(s)).cuda()
    resident = gpu_experts(s)
    host = _host_experts(qm, s)
    ring = qm.Ring(R, s.H, s.I)
    try:
        y = qm.strata_moe_prefill(x, wr, resident, s.K, torch.empty_like(x))
        for call in range(3):  # consecutive calls continue around the ring
            ys = qm.strata_moe_prefill_streamed(x, wr, host, ring, s.K, torch.empty_like(x))
            assert torch.equal(ys, y), f"call {call}"
        # the prepared router matrix as well
        ysp = qm.strata_moe_prefill_streamed(x, wr, host.with_prepared_router(wr), ring, s.K, torch.empty_like(x))
        assert torch.equal(ysp, y)
        torch.cuda.synchronize()
    finally:
        ring.close()


def test_streamed_layer_at_the_stream_all_chunk(qm):
    """1024 tokens over the 512 production-size experts (1.26 GB streamed per
    call) through a 96-slot ring."""
    s = S.shape("stream_all_1k")
    x = torch.from_numpy(S.activations(s)).cuda()
    wr = torch.from_numpy(S.router_weight(s)).cuda()
    resident = gpu_experts(s)
    host = _host_experts(qm, s)
    ring = qm.Ring(96, s.H, s.I)
    try:
        y = qm.strata_moe_prefill(x, wr, resident, s.K, torch.empty_like(x))
        for _ in range(2):
            ys = qm.strata_moe_prefill_streamed(x, wr, host, ring, s.K, torch.empty_like(x))
            assert torch.equal(ys, y)
        torch.cuda.synchronize()
    finally:
        ring.close()


def test_streamed_layer_rejects_a_resident_layout(qm):
    s = S.shape("tiny")
    ring = qm.Ring(4, s.H, s.I)
    try:
        x = torch.from_numpy(S.activations(s)).cuda()
        wr = torch.from_numpy(S.router_weight(s)).cuda()
        with pytest.raises(TypeError):
            qm.strata_moe_prefill_streamed(x, wr, gpu_experts(s), ring, s.K, torch.empty_like(x))
        other = qm.Ring(4, 384, s.I)
        try:
            with pytest.raises(ValueError):
                qm.strata_moe_prefill_streamed(x, wr, _host_experts(qm, s), other, s.K, torch.empty_like(x))
        finally:
            other.close()
    finally:
        ring.close()
