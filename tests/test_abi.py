"""The C ABI boundary without a GPU: the library loads, exports every entry
point include/strata_moe.h declares, sizes its buffers, and rejects bad
arguments on the host before anything would be enqueued."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "strata_moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(strata_moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def qm():
    import quantized_routed_expert_logits_amd as qm
    return qm


def test_header_declares_the_layer_entry_points():
    names = _declared()
    for n in ("strata_moe_prefill", "strata_moe_route", "strata_moe_group", "strata_moe_quantize",
              "strata_moe_gate_up", "strata_moe_down", "strata_moe_pack", "strata_moe_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(qm):
    lib = ctypes.CDLL(qm.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(qm.EXPORTED) == _declared()


def test_packed_sizes_are_two_bits_plus_fp16_scales(qm):
    gu, dn = qm.strata_moe_packed_bytes(2560, 1024)
    # 2 bits per weight + one fp16 per 32 weights, rounded up to 256 bytes
    assert gu == 2 * 1024 * 2560 * (2 / 8 + 2 / 32)
    assert dn == 2560 * 1024 * (2 / 8 + 2 / 32)
    assert gu + dn == 3 * 2560 * 1024 * 10 // 32  # 2.4576 MB per expert
    with pytest.raises(qm.StrataMoeError) as ei:
        qm.strata_moe_packed_bytes(2560, 1000)
    assert ei.value.code == qm.EINVAL


def _experts_struct(qm, E=512, H=2560, I=1024, fmt=1):
    try:
        gu, dn = qm.strata_moe_packed_bytes(H, I)
    except qm.StrataMoeError:
        gu = dn = 1 << 24
    return qm.ExpertsStruct(E, H, I, fmt, 1 << 20, gu, 1 << 30, dn, None)


def test_workspace_bytes_scale_with_tokens(qm):
    st = _experts_struct(qm)
    b = ctypes.c_size_t()
    lib = qm.library()
    assert lib.strata_moe_workspace_bytes(8192, 10, ctypes.byref(st), ctypes.byref(b)) == 0
    small = b.value
    assert lib.strata_moe_workspace_bytes(32768, 10, ctypes.byref(st), ctypes.byref(b)) == 0
    assert b.value > 3.5 * small
    # H codes as fp16 (n*I*2) dominate: at least that much
    assert small >= 8192 * 10 * 1024 * 2


@pytest.mark.parametrize("K,T,fmt,H,I,E,code", [
    (0, 8, 1, 2560, 1024, 512, -1),      # K < 1
    (17, 8, 1, 2560, 1024, 512, -1),     # K > 16
    (10, -1, 1, 2560, 1024, 512, -1),    # negative T
    (10, 8, 7, 2560, 1024, 512, -2),     # unknown format
    (10, 8, 1, 2600, 1024, 512, -1),     # H not a multiple of 128
    (10, 8, 1, 2624, 1024, 512, -1),     # H a multiple of 64 but not of 128
    (10, 8, 1, 2560, 1000, 512, -1),     # I not a multiple of 64
    (10, 8, 1, 2560, 1056, 512, -1),     # I a multiple of 32 but not of 64
    (10, 8, 1, 8192, 1024, 512, -1),     # H above 4096
    (10, 8, 1, 2560, 1024, 2048, -1),    # too many experts
    (4, 8, 1, 256, 128, 3, -1),          # K > E
])
def test_prefill_rejects_bad_arguments_on_the_host(qm, K, T, fmt, H, I, E, code):
    st = _experts_struct(qm, E=E, H=H, I=I, fmt=fmt)
    lib = qm.library()
    rc = lib.strata_moe_prefill(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(st), T, K,
                                ctypes.c_void_p(16), None)
    assert rc == code
    assert qm.strata_moe_last_error() != ""


def test_shared_expert_sizes_and_limits_on_the_host(qm):
    # a shared expert widens the grouping to K + 1 pairs of E + 1 experts
    lib = qm.library()
    b = ctypes.c_size_t()
    st = _experts_struct(qm)
    assert lib.strata_moe_workspace_bytes(8192, 10, ctypes.byref(st), ctypes.byref(b)) == 0
    plain = b.value
    st.shared_gate = 1 << 12
    assert lib.strata_moe_workspace_bytes(8192, 10, ctypes.byref(st), ctypes.byref(b)) == 0
    assert b.value >= plain + 8192 * 1024 * 2  # at least one more row of H codes per token
    for K, E in ((16, 512), (10, 1024)):  # no pair slot left; no expert index left
        st = _experts_struct(qm, E=E)
        st.shared_gate = 1 << 12
        rc = lib.strata_moe_prefill(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(st), 8, K,
                                    ctypes.c_void_p(16), None)
        assert rc == qm.EINVAL and "shared" in qm.strata_moe_last_error()
    st = _experts_struct(qm)
    st.shared_gate = (1 << 12) + 4  # not 16-byte aligned
    assert lib.strata_moe_workspace_bytes(8, 10, ctypes.byref(st), ctypes.byref(b)) == qm.EINVAL
    # the C struct's last fields: ctypes offsets after the router_prepared pointer
    assert qm.ExpertsStruct.shared_gate.offset == qm.ExpertsStruct.router_prepared.offset + ctypes.sizeof(ctypes.c_void_p)
    assert qm.ExpertsStruct.flags.offset == qm.ExpertsStruct.shared_gate.offset + ctypes.sizeof(ctypes.c_void_p)
    st = _experts_struct(qm)
    st.flags = 8  # no such flag
    assert lib.strata_moe_workspace_bytes(8, 10, ctypes.byref(st), ctypes.byref(b)) == qm.EINVAL


def test_prefill_rejects_short_strides_and_null(qm):
    lib = qm.library()
    st = _experts_struct(qm)
    st.gate_up_stride -= 256
    assert lib.strata_moe_prefill(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(st), 8, 10,
                                  ctypes.c_void_p(16), None) == qm.EINVAL
    assert lib.strata_moe_prefill(ctypes.c_void_p(16), ctypes.c_void_p(16), None, 8, 10,
                                  ctypes.c_void_p(16), None) == qm.EINVAL


def test_zero_tokens_is_a_no_op(qm):
    lib = qm.library()
    st = _experts_struct(qm)
    assert lib.strata_moe_prefill(None, None, ctypes.byref(st), 0, 10, None, None) == 0


def test_debug_entry_points_validate_sizes(qm):
    lib = qm.library()
    assert lib.strata_moe_quantize(ctypes.c_void_p(16), 4, 48, ctypes.c_void_p(16), ctypes.c_void_p(16), None) \
        == qm.EINVAL
    assert lib.strata_moe_route(ctypes.c_void_p(16), ctypes.c_void_p(16), None, 4, 2560, 2000, 10,
                                ctypes.c_void_p(16), ctypes.c_void_p(16), None) == qm.EINVAL
    assert lib.strata_moe_group(ctypes.c_void_p(16), 4, 12, 8, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                ctypes.c_void_p(16), None) == qm.EINVAL


def test_timing_names(qm):
    lib = qm.library()
    n = lib.strata_moe_timing_kinds()
    names = [lib.strata_moe_timing_name(i).decode() for i in range(n)]
    assert "gate_up" in names and "down" in names


def test_binding_rejects_mismatched_tensors_before_the_call(qm):
    """The C entry points take raw pointers and sizes; the binding checks every
    tensor's shape, dtype and device against the layer's sizes first and
    raises before the C call (CPU tensors here: nothing reaches a device)."""
    import torch

    E, H, I, T, K = 8, 256, 128, 4, 2
    ex = qm.Experts(E, H, I, device="cpu")
    x = torch.zeros((T, H))
    wr = torch.zeros((H, E))
    out = torch.zeros((T, H))
    bad_layer = [
        (torch.zeros((T, 384)), wr, out),     # x wider than the experts' hidden size
        (x, torch.zeros((H, E - 1)), out),    # router_w of another expert count
        (x, torch.zeros((E, H)), out),        # router_w transposed
        (x, wr, torch.zeros((T, I))),         # out of the wrong width
        (x, wr, torch.zeros((T + 1, H))),     # out of another token count
        (torch.zeros(T * H), wr, out),        # x not 2-D
    ]
    for xx, ww, oo in bad_layer:
        with pytest.raises(ValueError):
            qm.strata_moe_prefill(xx, ww, ex, K, oo)
        with pytest.raises(ValueError):
            qm.strata_moe_prefill_debug(xx, ww, ex, K, oo)
    with pytest.raises(TypeError):
        qm.strata_moe_prefill(x.double(), wr, ex, K, out)   # dtype
    with pytest.raises(TypeError):
        qm.strata_moe_prefill(x, wr, ex, K, out)            # right shapes, but not device tensors
    with pytest.raises(ValueError):
        ex.with_router_bias(torch.zeros(E + 1))
    with pytest.raises(ValueError):
        qm.strata_moe_route(x, wr, torch.zeros(E - 1), K)
    with pytest.raises(ValueError):
        qm.strata_moe_route(x, wr, None, K, ids=torch.zeros((T, K + 1), dtype=torch.int32))
    n = T * K
    qx, sx = torch.zeros((T, H), dtype=torch.int8), torch.zeros((T, H // 32))
    offsets, src = torch.zeros(E + 1, dtype=torch.int32), torch.zeros(n, dtype=torch.int32)
    with pytest.raises(ValueError):
        qm.strata_moe_gate_up(qx, torch.zeros((T, H // 16)), offsets, src, K, ex)
    with pytest.raises(ValueError):
        qm.strata_moe_gate_up(qx, sx, torch.zeros(E, dtype=torch.int32), src, K, ex)
    with pytest.raises(ValueError):
        qm.strata_moe_gate_up(qx, sx, offsets, torch.zeros(n - 1, dtype=torch.int32), K, ex)
    qh, sh = torch.zeros((n, I), dtype=torch.int8), torch.zeros((n, I // 32))
    slot, p = torch.zeros(n, dtype=torch.int32), torch.zeros((T, K))
    with pytest.raises(ValueError):
        qm.strata_moe_down(torch.zeros((n, H), dtype=torch.int8), sh, offsets, src, slot, p, ex, out)
    with pytest.raises(ValueError):
        qm.strata_moe_down(qh, sh, offsets, src, slot, p, ex, torch.zeros((T, I)))
    with pytest.raises(TypeError):
        qm.strata_moe_down(qh, sh, offsets, src, slot, p, ex, out)  # right shapes, CPU tensors


def test_ring_sizes_and_host_checks(qm):
    lib = qm.library()
    b = ctypes.c_size_t()
    assert lib.strata_moe_ring_bytes(96, 2560, 1024, ctypes.byref(b)) == 0
    gu, dn = qm.strata_moe_packed_bytes(2560, 1024)
    assert b.value == 96 * (gu + dn)  # one expert (gate/up + down) per slot
    assert lib.strata_moe_ring_bytes(0, 2560, 1024, ctypes.byref(b)) == qm.EINVAL
    h = ctypes.c_void_p()
    # no copy stream; too little slot memory; misaligned memory: rejected before any device call
    assert lib.strata_moe_ring_create(4, 256, 128, ctypes.c_void_p(1 << 20), 1 << 30, None, ctypes.byref(h)) \
        == qm.EINVAL
    assert lib.strata_moe_ring_create(4, 256, 128, ctypes.c_void_p(1 << 20), 256, ctypes.c_void_p(8),
                                      ctypes.byref(h)) == qm.EINVAL
    assert lib.strata_moe_ring_create(4, 256, 128, ctypes.c_void_p((1 << 20) + 8), 1 << 30, ctypes.c_void_p(8),
                                      ctypes.byref(h)) == qm.EINVAL
    assert lib.strata_moe_ring_destroy(None) == 0
    st = _experts_struct(qm)
    assert lib.strata_moe_prefill_streamed(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(st), None, 8, 10,
                                           ctypes.c_void_p(16), None) == qm.EINVAL


def test_noalloc_entry_point_checks_on_the_host(qm):
    lib = qm.library()
    st = _experts_struct(qm)
    # argument errors come back before the scratch array or any device is touched
    assert lib.strata_moe_prefill_noalloc(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.byref(st), 8, 0,
                                          ctypes.c_void_p(16), None) == qm.EINVAL
    assert lib.strata_moe_prefill_noalloc(None, None, ctypes.byref(st), 0, 10, None, None) == 0  # T = 0: no-op


def test_probe_library_exports_and_rejects_bad_arguments():
    from quantized_routed_expert_logits_amd import probe
    lib = ctypes.CDLL(probe.LIB_PATH)
    for name in ("strata_probe_mfma_rate", "strata_probe_scaled_blocks", "strata_probe_scaled_tiles",
                 "strata_probe_block_step", "strata_probe_mfma_f16", "strata_probe_hbm_read"):
        assert hasattr(lib, name), name
    d = ctypes.c_double()
    # argument checks come before any HIP call
    assert probe._lib.strata_probe_hbm_read(1000, 64, ctypes.byref(d), ctypes.byref(d)) == -1  # under 1 MiB
    assert probe._lib.strata_probe_hbm_read((1 << 20) + 8, 64, ctypes.byref(d), ctypes.byref(d)) == -1  # not 16 | bytes
    assert probe._lib.strata_probe_hbm_read(1 << 20, 0, ctypes.byref(d), ctypes.byref(d)) == -1
    assert probe._lib.strata_probe_mfma_rate(99, 1, 1, ctypes.byref(d), ctypes.byref(d)) == -1
    assert probe._lib.strata_probe_scaled_tiles(2, 6, 1, 1, ctypes.byref(d), ctypes.byref(d)) == -1  # form
    assert probe._lib.strata_probe_scaled_tiles(0, 4, 1, 1, ctypes.byref(d), ctypes.byref(d)) == -1  # tiles
    assert probe._lib.strata_probe_block_step(3, 1, 2, ctypes.byref(d), ctypes.byref(d)) == -1  # step
    assert probe._lib.strata_probe_block_step(0, 1, 3, ctypes.byref(d), ctypes.byref(d)) == -1  # odd blocks


def test_one_call_is_limited_by_its_tiled_operands(qm):
    """(T*K + 15*E) * max(H, I) * 2 bytes must stay below 2 GiB: about 41,000
    tokens at H = 2560, K = 10, E = 512; longer prompts run as several calls."""
    st = _experts_struct(qm)
    b = ctypes.c_size_t()
    lib = qm.library()
    assert lib.strata_moe_workspace_bytes(40000, 10, ctypes.byref(st), ctypes.byref(b)) == 0
    assert lib.strata_moe_workspace_bytes(42000, 10, ctypes.byref(st), ctypes.byref(b)) == qm.EINVAL
    assert "too large" in qm.strata_moe_last_error()
