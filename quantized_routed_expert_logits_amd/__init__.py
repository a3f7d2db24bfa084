"""Python binding of libstrata_moe (the MI355X routed-expert prompt MoE layer).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch provides device memory
and streams); each function takes the same arguments as the C entry point of
the same name in include/strata_moe.h, with shapes taken from the tensors
where the C call takes sizes.  There is no CPU fallback: importing this
package fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstrata_moe.so")

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
ENOMEM = -3
EHIP = -4
EDATA = -5
Q2_SYM = 1  # w = d * (q - 1.5)
Q2_0 = 2    # w = d * (q - 1), the pages' Q2_0 packs
FORMATS = {"q2_sym": Q2_SYM, "q2_0": Q2_0}
FLAG_NO_GEMV = 1        # every chunk to the MFMA kernels (no GEMV, also at decode-window sizes)
FLAG_PER_SLOT_Q8 = 2    # the GEMV's input rounded per routed slot in the q8_1 form (A/B arm)
FLAG_GEMV_ALWAYS = 4    # the GEMV takes chunks of <= 8 rows at any average rows per expert


class StrataMoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_i64, _i32 = ctypes.c_int64, ctypes.c_int32


class ExpertsStruct(ctypes.Structure):
    _fields_ = [("n_expert", _i32), ("hidden", _i32), ("ffn", _i32), ("format", _i32),
                ("gate_up", _P), ("gate_up_stride", _i64), ("down", _P), ("down_stride", _i64),
                ("router_bias", _P), ("router_prepared", _P), ("shared_gate", _P), ("flags", _i32)]


class DebugStruct(ctypes.Structure):
    _fields_ = [(name, _P) for name in ("ids", "p", "offsets", "src", "slot", "qx", "sx", "qh", "sh")]


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_sig("strata_moe_device_supported", [])
_sig("strata_moe_last_error", [], ctypes.c_char_p)
_sig("strata_moe_packed_bytes", [_i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)])
_sig("strata_moe_workspace_bytes", [_i64, _i32, ctypes.POINTER(ExpertsStruct), ctypes.POINTER(ctypes.c_size_t)])
_sig("strata_moe_set_workspace", [_P, ctypes.c_size_t])
_sig("strata_moe_router_prepared_bytes", [_i32, _i32, ctypes.POINTER(ctypes.c_size_t)])
_sig("strata_moe_prepare_router", [_P, _i32, _i32, _P, _P])
_sig("strata_moe_pack", [_P, _P, _P, _P, _i32, _i32, _i32, _i32, _P, _i64, _P, _i64, _P])
_sig("strata_moe_unpack", [_P, _i64, _P, _i64, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P])
_sig("strata_moe_prefill", [_P, _P, ctypes.POINTER(ExpertsStruct), _i64, _i32, _P, _P])
_sig("strata_moe_prefill_noalloc", [_P, _P, ctypes.POINTER(ExpertsStruct), _i64, _i32, _P, _P])
_sig("strata_moe_prefill_debug", [_P, _P, ctypes.POINTER(ExpertsStruct), _i64, _i32, _P,
                                  ctypes.POINTER(DebugStruct), _P])
_sig("strata_moe_route", [_P, _P, _P, _i64, _i32, _i32, _i32, _P, _P, _P])
_sig("strata_moe_group", [_P, _i64, _i32, _i32, _P, _P, _P, _P])
_sig("strata_moe_quantize", [_P, _i64, _i32, _P, _P, _P])
_sig("strata_moe_gate_up", [_P, _P, _P, _P, _i64, _i32, ctypes.POINTER(ExpertsStruct), _P, _P, _P])
_sig("strata_moe_down", [_P, _P, _P, _P, _P, _P, _i64, _i32, ctypes.POINTER(ExpertsStruct), _P, _P])
_sig("strata_moe_ring_bytes", [_i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)])
_sig("strata_moe_ring_create", [_i32, _i32, _i32, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)])
_sig("strata_moe_ring_destroy", [_P])
_sig("strata_moe_prefill_streamed", [_P, _P, ctypes.POINTER(ExpertsStruct), _P, _i64, _i32, _P, _P])
_sig("strata_moe_timing", [ctypes.c_int, _i32])
_sig("strata_moe_timing_kinds", [])
_sig("strata_moe_timing_name", [ctypes.c_int], ctypes.c_char_p)
_sig("strata_moe_timing_read", [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32), ctypes.c_int])

EXPORTED = [
    "strata_moe_device_supported", "strata_moe_last_error", "strata_moe_packed_bytes",
    "strata_moe_workspace_bytes", "strata_moe_set_workspace", "strata_moe_router_prepared_bytes",
    "strata_moe_prepare_router", "strata_moe_pack", "strata_moe_unpack",
    "strata_moe_prefill", "strata_moe_prefill_debug", "strata_moe_route", "strata_moe_group",
    "strata_moe_quantize", "strata_moe_gate_up", "strata_moe_down", "strata_moe_timing",
    "strata_moe_timing_kinds", "strata_moe_timing_name", "strata_moe_timing_read",
    "strata_moe_ring_bytes", "strata_moe_ring_create", "strata_moe_ring_destroy", "strata_moe_prefill_streamed",
    "strata_moe_prefill_noalloc",
]
NOALLOC_SCRATCH_BYTES = 512 << 20  # STRATA_MOE_NOALLOC_SCRATCH_BYTES


def library() -> ctypes.CDLL:
    return _lib


def strata_moe_last_error() -> str:
    return _lib.strata_moe_last_error().decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise StrataMoeError(rc, f"{what}: {strata_moe_last_error()}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("expected a CUDA (HIP) torch tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t, dt, name):
    if t is not None and t.dtype != dt:
        raise TypeError(f"{name} must be {dt}, got {t.dtype}")


def _expect(t, name: str, shape: tuple, dt):
    """Host-side check of one tensor argument before the C call: the library
    takes raw pointers and trusts the sizes it is given, so a tensor of the
    wrong shape would send its kernels past the allocation."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    _dtype(t, dt, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _one_device(**tensors):
    """Every given tensor is a CUDA (HIP) tensor, all on one device."""
    devs = set()
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"arguments are on different devices: {sorted(str(d) for d in devs)}")


def _check_layer_args(x, router_w, experts: "Experts", out):
    """x [T][H], router_w [H][E], out [T][H] (fp32), on the experts' device
    (streamed experts: their parameters' device; the blobs are in host memory)."""
    H, E = experts.hidden, experts.n_expert
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D [T][H] tensor")
    T = x.shape[0]
    _expect(x, "x", (T, H), torch.float32)
    _expect(router_w, "router_w", (H, E), torch.float32)
    _expect(out, "out", (T, H), torch.float32)
    blobs = {} if getattr(experts, "streamed", False) else dict(gate_up=experts.gate_up, down=experts.down)
    _one_device(x=x, router_w=router_w, out=out, router_bias=experts.router_bias,
                router_prepared=experts.router_prepared, shared_gate=experts.shared_gate, **blobs)
    return T


# ------------------------------------------------------------------- queries
def strata_moe_device_supported() -> bool:
    return bool(_lib.strata_moe_device_supported())


def strata_moe_packed_bytes(hidden: int, ffn: int) -> tuple[int, int]:
    gu, dn = _i64(), _i64()
    _check(_lib.strata_moe_packed_bytes(hidden, ffn, ctypes.byref(gu), ctypes.byref(dn)), "strata_moe_packed_bytes")
    return gu.value, dn.value


def strata_moe_router_prepared_bytes(hidden: int, n_expert: int) -> int:
    b = ctypes.c_size_t()
    _check(_lib.strata_moe_router_prepared_bytes(hidden, n_expert, ctypes.byref(b)), "strata_moe_router_prepared_bytes")
    return b.value


def strata_moe_prepare_router(router_w: torch.Tensor, stream=None) -> torch.Tensor:
    """router_w [H][E] fp32 on the device -> its prepared form (a uint8 device tensor)."""
    _dtype(router_w, torch.float32, "router_w")
    H, E = router_w.shape
    prepared = torch.empty(strata_moe_router_prepared_bytes(H, E), dtype=torch.uint8, device=router_w.device)
    _check(_lib.strata_moe_prepare_router(_ptr(router_w), H, E, _ptr(prepared), _stream(stream)),
           "strata_moe_prepare_router")
    return prepared


def strata_moe_set_workspace(buf: torch.Tensor | None) -> None:
    if buf is None:
        _check(_lib.strata_moe_set_workspace(None, 0), "strata_moe_set_workspace")
    else:
        _check(_lib.strata_moe_set_workspace(_ptr(buf), buf.numel() * buf.element_size()), "strata_moe_set_workspace")


# ------------------------------------------------------------------- experts
class Experts:
    """A layer's packed experts in device memory (blobs owned by torch).

    shared=True adds a blob slot for the layer's shared expert at index
    n_expert (pack it like a routed expert); the layer runs it once its scalar
    gate vector is set (with_shared_gate)."""

    def __init__(self, n_expert: int, hidden: int, ffn: int, router_bias: torch.Tensor | None = None,
                 device: str | torch.device = "cuda", fmt: str = "q2_sym", shared: bool = False):
        if fmt not in FORMATS:
            raise ValueError(f"unknown weight format {fmt!r}; one of {sorted(FORMATS)}")
        self.n_expert, self.hidden, self.ffn, self.format = n_expert, hidden, ffn, FORMATS[fmt]
        self.shared = bool(shared)
        nb = n_expert + self.shared
        self.gate_up_stride, self.down_stride = strata_moe_packed_bytes(hidden, ffn)
        self.gate_up = torch.empty(nb * self.gate_up_stride, dtype=torch.uint8, device=device)
        self.down = torch.empty(nb * self.down_stride, dtype=torch.uint8, device=device)
        if router_bias is not None:
            _expect(router_bias, "router_bias", (n_expert,), torch.float32)
        self.router_bias = router_bias
        self.router_prepared = None
        self.shared_gate = None
        self.flags = 0
        self._restruct()

    def _restruct(self):
        self.struct = ExpertsStruct(self.n_expert, self.hidden, self.ffn, self.format, self.gate_up.data_ptr(),
                                    self.gate_up_stride, self.down.data_ptr(), self.down_stride,
                                    None if self.router_bias is None else self.router_bias.data_ptr(),
                                    None if self.router_prepared is None else self.router_prepared.data_ptr(),
                                    None if self.shared_gate is None else self.shared_gate.data_ptr(),
                                    getattr(self, "flags", 0))

    def with_flags(self, flags: int) -> "Experts":
        """The same blobs with other kernel-choice flags (FLAG_NO_GEMV, FLAG_PER_SLOT_Q8, FLAG_GEMV_ALWAYS)."""
        import copy

        other = copy.copy(self)
        other.flags = int(flags)
        other._restruct()
        return other

    def with_router_bias(self, router_bias: torch.Tensor | None) -> "Experts":
        """The same blobs with another router bias (or none)."""
        import copy

        if router_bias is not None:
            _expect(router_bias, "router_bias", (self.n_expert,), torch.float32)
        other = copy.copy(self)
        other.router_bias = router_bias
        other._restruct()
        return other

    def with_shared_gate(self, gate: torch.Tensor | None) -> "Experts":
        """The same blobs with the shared expert's scalar gate vector [H] fp32
        (None: the layer runs the routed experts only)."""
        import copy

        if gate is not None:
            if not self.shared:
                raise ValueError("these experts have no shared-expert blob (Experts(..., shared=True))")
            _dtype(gate, torch.float32, "shared_gate")
            if tuple(gate.shape) != (self.hidden,) or not gate.is_contiguous():
                raise ValueError(f"shared_gate must be a contiguous [{self.hidden}] tensor")
        other = copy.copy(self)
        other.shared_gate = gate
        other._restruct()
        return other

    def with_prepared_router(self, router_w: torch.Tensor | None, stream=None) -> "Experts":
        """The same blobs with router_w prepared once (strata_moe_prepare_router);
        the layer calls must then pass the same router_w.  None: prepare per call."""
        import copy

        if router_w is not None:
            _expect(router_w, "router_w", (self.hidden, self.n_expert), torch.float32)
        other = copy.copy(self)
        other.router_prepared = None if router_w is None else strata_moe_prepare_router(router_w, stream)
        other._restruct()
        return other

    def pack(self, e0: int, codes_gu, scales_gu, codes_d, scales_d, stream=None):
        """Pack experts [e0, e0 + len(codes_gu)) from canonical arrays (numpy
        or torch; copied to the device if needed)."""
        dev = self.gate_up.device

        def to_dev(a, dt):
            if isinstance(a, np.ndarray):
                a = torch.from_numpy(np.ascontiguousarray(a))
            return a.to(device=dev, dtype=dt).contiguous()

        cg, sg = to_dev(codes_gu, torch.uint8), to_dev(scales_gu.view(np.int16) if isinstance(scales_gu, np.ndarray)
                                                       else scales_gu, torch.int16)
        cd, sd = to_dev(codes_d, torch.uint8), to_dev(scales_d.view(np.int16) if isinstance(scales_d, np.ndarray)
                                                      else scales_d, torch.int16)
        ne = cg.shape[0]
        assert cg.shape == (ne, 2 * self.ffn, self.hidden) and cd.shape == (ne, self.hidden, self.ffn)
        strata_moe_pack(cg, sg, cd, sd, e0, e0 + ne, self.hidden, self.ffn, self.gate_up, self.gate_up_stride,
                        self.down, self.down_stride, stream)


def strata_moe_pack(codes_gu, scales_gu, codes_d, scales_d, e0, e1, hidden, ffn, gate_up, gate_up_stride, down,
                    down_stride, stream=None):
    _check(_lib.strata_moe_pack(_ptr(codes_gu), _ptr(scales_gu), _ptr(codes_d), _ptr(scales_d), e0, e1, hidden, ffn,
                                _ptr(gate_up), gate_up_stride, _ptr(down), down_stride, _stream(stream)),
           "strata_moe_pack")


def strata_moe_unpack(experts: Experts, e0: int, e1: int, stream=None):
    """Returns canonical (codes_gu, scales_gu, codes_d, scales_d) device tensors of experts [e0, e1)."""
    ne, H, I = e1 - e0, experts.hidden, experts.ffn
    dev = experts.gate_up.device
    cg = torch.empty((ne, 2 * I, H), dtype=torch.uint8, device=dev)
    sg = torch.empty((ne, 2 * I, H // 32), dtype=torch.int16, device=dev)
    cd = torch.empty((ne, H, I), dtype=torch.uint8, device=dev)
    sd = torch.empty((ne, H, I // 32), dtype=torch.int16, device=dev)
    _check(_lib.strata_moe_unpack(_ptr(experts.gate_up), experts.gate_up_stride, _ptr(experts.down),
                                  experts.down_stride, e0, e1, H, I, _ptr(cg), _ptr(sg), _ptr(cd), _ptr(sd),
                                  _stream(stream)), "strata_moe_unpack")
    return cg, sg, cd, sd


def strata_moe_workspace_bytes(T: int, K: int, experts: Experts) -> int:
    b = ctypes.c_size_t()
    _check(_lib.strata_moe_workspace_bytes(T, K, ctypes.byref(experts.struct), ctypes.byref(b)),
           "strata_moe_workspace_bytes")
    return b.value


# ---------------------------------------------------------- streamed experts
class HostExperts(Experts):
    """A layer's packed experts in pinned host memory, for the streamed layer:
    expert e's gate/up blob at e * S and its down blob right after it (S =
    one ring slot), the layout strata_moe_prefill_streamed reads.  Packing
    runs on `device` (the library's packer) and the result is copied here."""

    streamed = True

    def __init__(self, n_expert: int, hidden: int, ffn: int, router_bias: torch.Tensor | None = None,
                 device: str | torch.device = "cuda", fmt: str = "q2_sym", shared: bool = False):
        if fmt not in FORMATS:
            raise ValueError(f"unknown weight format {fmt!r}; one of {sorted(FORMATS)}")
        self.n_expert, self.hidden, self.ffn, self.format = n_expert, hidden, ffn, FORMATS[fmt]
        self.shared = bool(shared)
        self.device = torch.device(device)
        gu, dn = strata_moe_packed_bytes(hidden, ffn)
        self.gate_up_bytes, self.slot_bytes = gu, gu + dn
        self.gate_up_stride = self.down_stride = self.slot_bytes
        nb = n_expert + self.shared
        self.host = torch.empty(nb * self.slot_bytes, dtype=torch.uint8, pin_memory=True)
        self.gate_up = self.host
        self.down = self.host[gu:]
        if router_bias is not None:
            _expect(router_bias, "router_bias", (n_expert,), torch.float32)
        self.router_bias = router_bias
        self.router_prepared = None
        self.shared_gate = None
        self.flags = 0
        self._restruct()

    def pack(self, e0: int, codes_gu, scales_gu, codes_d, scales_d, stream=None):
        """Pack experts [e0, e0 + len(codes_gu)) from canonical arrays on the
        device, then copy the blobs into their host places."""
        ne = len(codes_gu)
        staging = torch.empty(ne * self.slot_bytes, dtype=torch.uint8, device=self.device)

        def to_dev(a, dt):
            if isinstance(a, np.ndarray):
                a = torch.from_numpy(np.ascontiguousarray(a))
            return a.to(device=self.device, dtype=dt).contiguous()

        as_i16 = lambda a: a.view(np.int16) if isinstance(a, np.ndarray) else a  # noqa: E731
        cg, sg = to_dev(codes_gu, torch.uint8), to_dev(as_i16(scales_gu), torch.int16)
        cd, sd = to_dev(codes_d, torch.uint8), to_dev(as_i16(scales_d), torch.int16)
        assert cg.shape == (ne, 2 * self.ffn, self.hidden) and cd.shape == (ne, self.hidden, self.ffn)
        strata_moe_pack(cg, sg, cd, sd, 0, ne, self.hidden, self.ffn, staging, self.slot_bytes,
                        staging[self.gate_up_bytes:], self.slot_bytes, stream)
        self.host[e0 * self.slot_bytes:(e0 + ne) * self.slot_bytes].copy_(staging)


class Ring:
    """A ring of n_slots device slots (torch memory) with a copy stream of its
    own (default priority) and the library's ring object over them."""

    def __init__(self, n_slots: int, hidden: int, ffn: int, device: str | torch.device = "cuda"):
        b = ctypes.c_size_t()
        _check(_lib.strata_moe_ring_bytes(n_slots, hidden, ffn, ctypes.byref(b)), "strata_moe_ring_bytes")
        self.n_slots, self.hidden, self.ffn = n_slots, hidden, ffn
        self.slots = torch.empty(b.value, dtype=torch.uint8, device=device)
        self.copy_stream = torch.cuda.Stream(device=device)
        h = _P()
        _check(_lib.strata_moe_ring_create(n_slots, hidden, ffn, _ptr(self.slots), b.value,
                                           ctypes.c_void_p(self.copy_stream.cuda_stream), ctypes.byref(h)),
               "strata_moe_ring_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _lib.strata_moe_ring_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover (interpreter shutdown)
            pass


def strata_moe_prefill_streamed(x: torch.Tensor, router_w: torch.Tensor, experts: HostExperts, ring: Ring, K: int,
                                out: torch.Tensor, stream=None) -> torch.Tensor:
    if not isinstance(experts, HostExperts):
        raise TypeError("streamed experts live in pinned host memory: use HostExperts")
    T = _check_layer_args(x, router_w, experts, out)
    if ring.handle is None:
        raise ValueError("the ring is closed")
    if (ring.hidden, ring.ffn) != (experts.hidden, experts.ffn):
        raise ValueError("the ring was made for other expert sizes")
    if ring.slots.device != x.device:
        raise ValueError("the ring is on another device")
    _check(_lib.strata_moe_prefill_streamed(_ptr(x), _ptr(router_w), ctypes.byref(experts.struct), ring.handle, T, K,
                                            _ptr(out), _stream(stream)), "strata_moe_prefill_streamed")
    return out


# --------------------------------------------------------------------- layer
def strata_moe_prefill(x: torch.Tensor, router_w: torch.Tensor, experts: Experts, K: int, out: torch.Tensor,
                       stream=None) -> torch.Tensor:
    T = _check_layer_args(x, router_w, experts, out)
    _check(_lib.strata_moe_prefill(_ptr(x), _ptr(router_w), ctypes.byref(experts.struct), T, K, _ptr(out),
                                   _stream(stream)), "strata_moe_prefill")
    return out


def strata_moe_prefill_noalloc(x: torch.Tensor, router_w: torch.Tensor, experts: Experts, K: int, out: torch.Tensor,
                               stream=None) -> torch.Tensor:
    """strata_moe_prefill on the library's fixed scratch: no device allocation."""
    T = _check_layer_args(x, router_w, experts, out)
    _check(_lib.strata_moe_prefill_noalloc(_ptr(x), _ptr(router_w), ctypes.byref(experts.struct), T, K, _ptr(out),
                                           _stream(stream)), "strata_moe_prefill_noalloc")
    return out


def strata_moe_prefill_debug(x, router_w, experts: Experts, K: int, out, stream=None) -> dict:
    """The layer plus its intermediates (ids, p, offsets, src, slot, qx, sx, qh, sh) as device tensors."""
    _check_layer_args(x, router_w, experts, out)
    T, H = x.shape
    sh = experts.shared_gate is not None  # the shared expert: pair slot K of each token, expert n_expert
    Kg = K + sh
    E, I, n = experts.n_expert + sh, experts.ffn, x.shape[0] * Kg
    dev = x.device
    d = dict(ids=torch.empty((T, Kg), dtype=torch.int32, device=dev),
             p=torch.empty((T, Kg), dtype=torch.float32, device=dev),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
             src=torch.empty(n, dtype=torch.int32, device=dev),
             slot=torch.empty(n, dtype=torch.int32, device=dev),
             qx=torch.empty((T, H), dtype=torch.int8, device=dev),
             sx=torch.empty((T, H // 32), dtype=torch.float32, device=dev),
             qh=torch.empty((n, I), dtype=torch.int8, device=dev),
             sh=torch.empty((n, I // 32), dtype=torch.float32, device=dev))
    dbg = DebugStruct(*[d[k].data_ptr() for k in ("ids", "p", "offsets", "src", "slot", "qx", "sx", "qh", "sh")])
    _check(_lib.strata_moe_prefill_debug(_ptr(x), _ptr(router_w), ctypes.byref(experts.struct), T, K, _ptr(out),
                                         ctypes.byref(dbg), _stream(stream)), "strata_moe_prefill_debug")
    d["out"] = out
    return d


# -------------------------------------------------------------- single steps
def strata_moe_route(x, router_w, bias, K: int, ids=None, p=None, stream=None):
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not isinstance(router_w, torch.Tensor) or router_w.dim() != 2:
        raise ValueError("x must be [T][H] and router_w [H][E]")
    T, H = x.shape
    E = router_w.shape[1]
    _expect(x, "x", (T, H), torch.float32)
    _expect(router_w, "router_w", (H, E), torch.float32)
    if bias is not None:
        _expect(bias, "bias", (E,), torch.float32)
    if ids is not None:
        _expect(ids, "ids", (T, K), torch.int32)
    if p is not None:
        _expect(p, "p", (T, K), torch.float32)
    _one_device(x=x, router_w=router_w, bias=bias, ids=ids, p=p)
    ids = torch.empty((T, K), dtype=torch.int32, device=x.device) if ids is None else ids
    p = torch.empty((T, K), dtype=torch.float32, device=x.device) if p is None else p
    _check(_lib.strata_moe_route(_ptr(x), _ptr(router_w), _ptr(bias), T, H, E, K, _ptr(ids), _ptr(p),
                                 _stream(stream)), "strata_moe_route")
    return ids, p


def strata_moe_group(ids, E: int, stream=None):
    if not isinstance(ids, torch.Tensor) or ids.dim() != 2:
        raise ValueError("ids must be a 2-D [T][K] tensor")
    _dtype(ids, torch.int32, "ids")
    _one_device(ids=ids)
    T, K = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    src = torch.empty(T * K, dtype=torch.int32, device=dev)
    slot = torch.empty(T * K, dtype=torch.int32, device=dev)
    _check(_lib.strata_moe_group(_ptr(ids), T, K, E, _ptr(offsets), _ptr(src), _ptr(slot), _stream(stream)),
           "strata_moe_group")
    return offsets, src, slot


def strata_moe_quantize(v, stream=None):
    if not isinstance(v, torch.Tensor) or v.dim() != 2:
        raise ValueError("v must be a 2-D [rows][cols] tensor")
    _dtype(v, torch.float32, "v")
    _one_device(v=v)
    rows, cols = v.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=v.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.float32, device=v.device)
    _check(_lib.strata_moe_quantize(_ptr(v), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)),
           "strata_moe_quantize")
    return codes, scales


def strata_moe_gate_up(qx, sx, offsets, src, K: int, experts: Experts, stream=None):
    if not isinstance(qx, torch.Tensor) or qx.dim() != 2:
        raise ValueError("qx must be a 2-D [T][H] tensor")
    T = qx.shape[0]
    n, I, H, E = T * K, experts.ffn, experts.hidden, experts.n_expert
    _expect(qx, "qx", (T, H), torch.int8)
    _expect(sx, "sx", (T, H // 32), torch.float32)
    _expect(offsets, "offsets", (E + 1,), torch.int32)
    _expect(src, "src", (n,), torch.int32)
    _one_device(qx=qx, sx=sx, offsets=offsets, src=src, gate_up=experts.gate_up)
    qh = torch.empty((n, I), dtype=torch.int8, device=qx.device)
    sh = torch.empty((n, I // 32), dtype=torch.float32, device=qx.device)
    _check(_lib.strata_moe_gate_up(_ptr(qx), _ptr(sx), _ptr(offsets), _ptr(src), T, K, ctypes.byref(experts.struct),
                                   _ptr(qh), _ptr(sh), _stream(stream)), "strata_moe_gate_up")
    return qh, sh


def strata_moe_down(qh, sh, offsets, src, slot, p, experts: Experts, out, stream=None):
    if not isinstance(p, torch.Tensor) or p.dim() != 2:
        raise ValueError("p must be a 2-D [T][K] tensor")
    T, K = p.shape
    n, I, H, E = T * K, experts.ffn, experts.hidden, experts.n_expert
    _expect(qh, "qh", (n, I), torch.int8)
    _expect(sh, "sh", (n, I // 32), torch.float32)
    _expect(offsets, "offsets", (E + 1,), torch.int32)
    _expect(src, "src", (n,), torch.int32)
    _expect(slot, "slot", (n,), torch.int32)
    _expect(p, "p", (T, K), torch.float32)
    _expect(out, "out", (T, H), torch.float32)
    _one_device(qh=qh, sh=sh, offsets=offsets, src=src, slot=slot, p=p, out=out, down=experts.down)
    _check(_lib.strata_moe_down(_ptr(qh), _ptr(sh), _ptr(offsets), _ptr(src), _ptr(slot), _ptr(p), T, K,
                                ctypes.byref(experts.struct), _ptr(out), _stream(stream)), "strata_moe_down")
    return out


# -------------------------------------------------------------------- timing
def strata_moe_timing(enable: bool, max_calls: int = 0) -> None:
    _check(_lib.strata_moe_timing(int(enable), max_calls), "strata_moe_timing")


def strata_moe_timing_read() -> dict:
    """{kernel kind: (total ms, launches)} of the current timing session."""
    n = _lib.strata_moe_timing_kinds()
    ms = (ctypes.c_double * n)()
    cnt = (_i32 * n)()
    _check(_lib.strata_moe_timing_read(ms, cnt, n), "strata_moe_timing_read")
    return {_lib.strata_moe_timing_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}
