"""CPU oracle of the routed-expert prompt MoE layer (double precision).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The HIP library and
its Python binding never import, load or call it, and the two share no code:
the only module both sides read is ``synthetic`` (the seeded input draws).

The arithmetic lives in ``strata_oracle.c`` (plain C, double precision, one
function per step of the layer, each citing the passage of the Strata pages it
follows); this wrapper marshals numpy arrays and chains the steps in the order
the pages give them (Winery-Strata prefill.cpp page, Prefill::run, MoE half:
router -> route -> quantize -> group -> experts -> combine).  The one step
written here in numpy (double) is the shared expert's gate and weighted sum
(s1, s2: the shared expert), built from the C steps.

Parity is pinned by ``tests/test_oracle_pins.py`` (brute force, closed forms,
invariants and exact round-trips); no function here is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "strata_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

BLOCK = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.oracle_router_logits.argtypes = [P, P, P, i64, i32, i32, P]
    lib.oracle_topk_softmax.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_group.argtypes = [P, i64, i32, i32, P, P, P]
    lib.oracle_group.restype = ctypes.c_int
    lib.oracle_quantize.argtypes = [P, i64, i32, P, P]
    lib.oracle_expert_rows.argtypes = [P, P, P, P, i32, i32, ctypes.c_double, i64, P, P, P, P, P, P]
    lib.oracle_combine.argtypes = [P, P, P, i64, i32, i32, P]
    lib.oracle_rows_multi.argtypes = [P, P, P, P, P, i32, i32, ctypes.c_double, i64, P, P, P, P, P, P]
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def half_to_double(bits: int) -> float:
    return float(_load().oracle_half_to_double(int(bits)))


def router_logits(x, wr, bias=None) -> np.ndarray:
    """c1: logits [T][E] in double (compensated sum), plus the bias if given."""
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    T, H = x.shape
    E = wr.shape[1]
    assert wr.shape[0] == H
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float64)
    _load().oracle_router_logits(_p(x), _p(wr), _p(b), T, H, E, _p(out))
    return out


def topk_softmax(logits, K: int):
    """c2: ids [T][K] int32 (rank order, ties -> lower index), p [T][K] double."""
    logits = _c(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    p = np.empty((T, K), np.float64)
    _load().oracle_topk_softmax(_p(logits), T, E, K, _p(ids), _p(p))
    return ids, p


def group(ids, E: int):
    """c3: offsets [E+1], src [T*K], slot [T*K] (stable counting sort)."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    offsets = np.empty(E + 1, np.int32)
    src = np.empty(T * K, np.int32)
    slot = np.empty(T * K, np.int32)
    rc = _load().oracle_group(_p(ids), T, K, E, _p(offsets), _p(src), _p(slot))
    if rc != 0:
        raise ValueError("routed id out of range")
    return offsets, src, slot


def quantize(v):
    """c4: per-32 int8 rounding of fp32 rows -> (codes int8, scales fp32)."""
    v = _c(v, np.float32)
    rows, cols = v.shape
    assert cols % BLOCK == 0
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows, cols // BLOCK), np.float32)
    _load().oracle_quantize(_p(v), rows, cols, _p(q), _p(s))
    return q, s


def code_zero(fmt: str) -> float:
    """The 2-bit map's offset z in w = d * (q - z): 1.5 for the symmetric map,
    1 for the pages' Q2_0 packs (Strata compare page, moe_fused.hpp header
    comment)."""
    return {"q2_sym": 1.5, "q2_0": 1.0}[fmt]


def expert_rows(ex, qx, sx, want_h: bool = False, fmt: str = "q2_sym"):
    """c5..c7 for one expert's routed rows.

    ex: an object with codes_gu [2I][H], scales_gu, codes_d [H][I], scales_d
    (``synthetic.Expert``); fmt: the weight map (code_zero).  Returns
    (h or None, qh, sh, D)."""
    cgu = _c(ex.codes_gu, np.uint8)
    sgu = _c(ex.scales_gu, np.uint16)
    cd = _c(ex.codes_d, np.uint8)
    sd = _c(ex.scales_d, np.uint16)
    H = cgu.shape[1]
    I = cgu.shape[0] // 2
    qx = _c(qx, np.int8).reshape(-1, H)
    sx = _c(sx, np.float32).reshape(-1, H // BLOCK)
    n = qx.shape[0]
    h = np.empty((n, I), np.float64) if want_h else None
    qh = np.empty((n, I), np.int8)
    sh = np.empty((n, I // BLOCK), np.float32)
    D = np.empty((n, H), np.float64)
    if n:
        _load().oracle_expert_rows(_p(cgu), _p(sgu), _p(cd), _p(sd), H, I, code_zero(fmt), n, _p(qx), _p(sx),
                                   _p(h), _p(qh), _p(sh), _p(D))
    return h, qh, sh, D


def combine(D, p, slot):
    """c8: y [T][H] = sum_k p[t][k] * D[slot[t*K+k]] in double."""
    D = _c(D, np.float64)
    p = _c(p, np.float64)
    slot = _c(slot, np.int32)
    T, K = p.shape
    H = D.shape[1]
    y = np.empty((T, H), np.float64)
    _load().oracle_combine(_p(D), _p(p), _p(slot), T, K, H, _p(y))
    return y


def shared_gate(x, wg) -> np.ndarray:
    """s1: the shared expert's scalar gate per token, g = sigmoid(x . wg), in
    double (the dot is c1's compensated sum with wg as the one column).  The
    pages compute this projection beside the shared expert in the MoE half of
    Prefill::run (prefill.cpp page) but do not print how it is applied; the
    reading here is the sigmoid-gated sum of s2."""
    s = router_logits(x, np.asarray(wg, np.float32).reshape(-1, 1))[:, 0]
    return 1.0 / (1.0 + np.exp(-s))


def _shared_term(shared, qx, sx, x, want_h, fmt):
    """s2: the shared expert's rows for every given token (the routed
    experts' c5..c7 on the token's int8 input) and its gate; y gains g * D."""
    ex, wg = shared
    h, qh, sh, D = expert_rows(ex, qx, sx, want_h, fmt)
    return dict(g=shared_gate(x, wg), qh=qh, sh=sh, h=h, D=D)


def layer(x, wr, bias, get_expert, E: int, K: int, want_h: bool = False, fmt: str = "q2_sym",
          shared=None) -> dict:
    """The whole layer on every token, all intermediates returned.

    get_expert(e) returns expert e's canonical arrays.  Steps in the pages'
    order: router logits, route (top-K + softmax), int8 activations once per
    token, grouping, per expert its rows (gate/up, SwiGLU, int8 H, down), and
    the combine.  shared = (expert arrays, gate vector [H]) adds the shared
    expert on every token, weighted by its scalar gate (s1, s2); its
    intermediates come back under "shared"."""
    T, H = x.shape
    logits = router_logits(x, wr, bias)
    ids, p = topk_softmax(logits, K)
    qx, sx = quantize(x)
    offsets, src, slot = group(ids, E)
    n = T * K
    ex0 = get_expert(0)
    I = ex0.codes_gu.shape[0] // 2
    qh = np.zeros((n, I), np.int8)
    sh = np.zeros((n, I // BLOCK), np.float32)
    h = np.zeros((n, I), np.float64) if want_h else None
    D = np.zeros((n, H), np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows = src[r0:r1]
        he, qhe, she, De = expert_rows(get_expert(e), qx[rows], sx[rows], want_h, fmt)
        qh[r0:r1], sh[r0:r1], D[r0:r1] = qhe, she, De
        if want_h:
            h[r0:r1] = he
    y = combine(D, p, slot)
    sh_term = None
    if shared is not None:
        sh_term = _shared_term(shared, qx, sx, x, want_h, fmt)
        y = y + sh_term["g"][:, None] * sh_term["D"]
    return dict(logits=logits, ids=ids, p=p, qx=qx, sx=sx, offsets=offsets, src=src, slot=slot,
                qh=qh, sh=sh, h=h, D=D, y=y, shared=sh_term)


def rows_multi(experts: list, which, qx, sx, fmt: str = "q2_sym", want_h: bool = False):
    """c5..c7 for rows of several experts: row r goes through experts[which[r]].
    Returns (qh, sh, D), plus h (the exact SwiGLU output, double) first if
    want_h."""
    keep = [(_c(e.codes_gu, np.uint8), _c(e.scales_gu, np.uint16), _c(e.codes_d, np.uint8),
             _c(e.scales_d, np.uint16)) for e in experts]
    H = keep[0][0].shape[1]
    I = keep[0][0].shape[0] // 2
    tables = [(ctypes.c_void_p * len(keep))(*[k[j].ctypes.data for k in keep]) for j in range(4)]
    which = _c(which, np.int32)
    qx = _c(qx, np.int8).reshape(-1, H)
    sx = _c(sx, np.float32).reshape(-1, H // BLOCK)
    n = qx.shape[0]
    qh = np.empty((n, I), np.int8)
    sh = np.empty((n, I // BLOCK), np.float32)
    D = np.empty((n, H), np.float64)
    h = np.empty((n, I), np.float64) if want_h else None
    if n:
        _load().oracle_rows_multi(tables[0], tables[1], tables[2], tables[3], _p(which), H, I, code_zero(fmt), n,
                                  _p(qx), _p(sx), _p(h), _p(qh), _p(sh), _p(D))
    return (h, qh, sh, D) if want_h else (qh, sh, D)


def layer_tokens(x, wr, bias, get_expert, K: int, tokens, fmt: str = "q2_sym", shared=None) -> dict:
    """The layer's output for a sample of tokens only.

    Every step of the layer is independent across tokens except the grouping,
    which only orders rows; so each sampled token is routed, quantized and
    pushed through its K experts on its own, and y[t] is exactly the full
    layer's y[t].  Returns per sampled token: ids, p, qx, sx, the K H-code
    rows, their scales, the exact SwiGLU outputs h they round and y."""
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = x[tokens]
    logits = router_logits(xs, wr, bias)
    ids, p = topk_softmax(logits, K)
    qx, sx = quantize(xs)
    S = len(tokens)
    H = x.shape[1]
    used = sorted(set(int(e) for e in ids.reshape(-1)))
    slot_of = {e: i for i, e in enumerate(used)}
    which = np.array([slot_of[int(e)] for e in ids.reshape(-1)], np.int32)
    # pairs token-major: row s*K + k is token s through its k-th expert
    rows = np.repeat(np.arange(S), K)
    h, qh, sh, D = rows_multi([get_expert(e) for e in used], which, qx[rows], sx[rows], fmt, want_h=True)
    I = qh.shape[1]
    # c8 with the pairs laid out token-major: row s*K + k holds D of (s, k)
    y = combine(D, p, np.arange(S * K, dtype=np.int32))
    D = D.reshape(S, K, H)
    qh = qh.reshape(S, K, I)
    sh = sh.reshape(S, K, I // BLOCK)
    h = h.reshape(S, K, I)
    sh_term = None
    if shared is not None:
        sh_term = _shared_term(shared, qx, sx, xs, False, fmt)
        y = y + sh_term["g"][:, None] * sh_term["D"]
    return dict(tokens=tokens, logits=logits, ids=ids, p=p, qx=qx, sx=sx, qh=qh, sh=sh, h=h, D=D, y=y,
                shared=sh_term)
