#!/usr/bin/env python3
"""Benchmark of the routed-expert prompt MoE layer on one MI355X.

A step is one strata_moe_prefill call -- router, top-K, grouping, int8
quantization, gate/up + SwiGLU + int8 H, down + weighted scatter-add -- over a
chunk of T tokens whose inputs, packed experts and prepared router matrix
(strata_moe_prepare_router, once, like the packing; --router-per-call prepares
it inside every step instead) are already resident in HBM.  Default workload: T = 8192, H = 2560, E = 512 experts, top-10, expert FFN
I = 1024, seeded synthetic inputs (the pages' own prompts and trained pack are
not available).

Prints one JSON line on stdout (progress goes to stderr):
  value        tokens/s of the layer over the timed steps (one GPU)
  roofline     the dominant kernel's achieved rate against its peak, measured
               with HIP events on the launch stream over the timed steps
  cpu_baseline the CPU oracle (double precision) timed on this host on a
               bounded sample of the same workload

    python bench.py [--steps K] [--warmup W] [--workload chunk_8k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE prefill layer tokens/s at T=8192 (512 exp, top-10); % int8 MFMA / HBM peak"
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="chunk_8k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--router-per-call", action="store_true",
                    help="prepare the router matrix inside every layer call instead of once with the experts")
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="tokens in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB after flushing the Infinity Cache "
                         "(counter calibration)")
    return ap.parse_args()


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in ("k_experts.hip", "internal.h"):
        with open(os.path.join(ROOT, "quantized_routed_expert_logits_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """Per-launch HBM bytes of `kernel` from the committed rocprofv3 counter
    summary, or None if there is none for the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures the layer on one GPU; --gpus {args.gpus} is not supported (the layer is "
              "data-parallel over token chunks with no exchange, so N GPUs run N independent chunks).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import quantized_routed_expert_logits_amd as qm
    import synthetic as S

    s = S.shape(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if not qm.strata_moe_device_supported():
        log("device is not gfx950")
        return 3

    log(f"workload {s.name}: T={s.T} H={s.H} E={s.E} K={s.K} I={s.I}; generating and packing experts")
    t_gen = time.time()
    canon = {}
    experts = qm.Experts(s.E, s.H, s.I, device=dev, fmt=s.fmt, shared=s.shared)
    chunk = 32
    nb = s.E + s.shared  # a shared expert is the last blob
    for e0 in range(0, nb, chunk):
        parts = [S.expert(s, e, args.seed) for e in range(e0, min(nb, e0 + chunk))]
        for i, p in enumerate(parts):
            canon[e0 + i] = p
        experts.pack(e0, np.stack([p.codes_gu for p in parts]), np.stack([p.scales_gu for p in parts]),
                     np.stack([p.codes_d for p in parts]), np.stack([p.scales_d for p in parts]))
    bias_np = S.router_bias(s, args.seed)
    bias = None if bias_np is None else torch.from_numpy(bias_np).to(dev)
    experts = experts.with_router_bias(bias)
    wg_np = S.shared_gate_weight(s, args.seed) if s.shared else None
    if s.shared:
        experts = experts.with_shared_gate(torch.from_numpy(wg_np).to(dev))
    x_np, wr_np = S.activations(s, args.seed), S.router_weight(s, args.seed)
    x = torch.from_numpy(x_np).to(dev)
    wr = torch.from_numpy(wr_np).to(dev)
    if not args.router_per_call:  # a layer parameter, prepared once like the packed experts
        experts = experts.with_prepared_router(wr)
    out = torch.empty_like(x)
    ws = torch.empty(qm.strata_moe_workspace_bytes(s.T, s.K, experts), dtype=torch.uint8, device=dev)
    qm.strata_moe_set_workspace(ws)
    torch.cuda.synchronize()
    log(f"inputs resident ({time.time() - t_gen:.1f}s); warmup {args.warmup}")

    for _ in range(args.warmup):
        qm.strata_moe_prefill(x, wr, experts, s.K, out)
    dbg_ids = qm.strata_moe_prefill_debug(x, wr, experts, s.K, out)["ids"]  # routing of this chunk (hit experts)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    qm.strata_moe_timing(True, args.steps)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        qm.strata_moe_prefill(x, wr, experts, s.K, out)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kt = qm.strata_moe_timing_read()
    qm.strata_moe_timing(False)
    qm.strata_moe_set_workspace(None)
    kernel_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in kt.items()}
    log(f"{ms_per_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}); per kernel "
        + ", ".join(f"{k} {v:.3f}" for k, v in kernel_ms.items()))

    if args.copy_probe_mib:
        a = torch.empty((args.copy_probe_mib << 20) // 4, dtype=torch.float32, device=dev).uniform_()
        b = torch.empty_like(a)
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        flush.fill_(1.0)  # 512 MiB written: evicts the 256 MiB Infinity Cache
        torch.cuda.synchronize()
        torch.neg(a, out=b)  # reads and writes copy_probe_mib MiB
        torch.cuda.synchronize()
        del flush
        log(f"copy probe: {args.copy_probe_mib} MiB")

    n = s.T * (s.K + s.shared)  # grouped rows: K routed pairs per token, plus the shared expert's
    flops = {"gate_up": 2.0 * n * 2 * s.I * s.H, "down": 2.0 * n * s.H * s.I}
    dominant = max(kernel_ms, key=kernel_ms.get)
    traffic = measured_traffic(dominant, s.name) if dominant in flops else None
    if dominant in flops and n / s.E >= 64:
        # many rows per expert: the grouped GEMM is a dense contraction
        achieved = flops[dominant] / (kernel_ms[dominant] * 1e-3) / 1e12
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic}
    elif dominant in flops:
        # few rows per expert: the GEMM streams the hit experts' packed weights once
        hit = int((torch.bincount(dbg_ids.reshape(-1).long(), minlength=s.E + s.shared) > 0).sum())
        rows = 2 * s.I if dominant == "gate_up" else s.H
        kd = s.H if dominant == "gate_up" else s.I
        wbytes = hit * rows * kd * (2 / 8 + 2 / 32)
        achieved = wbytes / (kernel_ms[dominant] * 1e-3) / 1e9
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": None, "traffic": None}

    cpu = None
    if args.cpu_tokens > 0:
        import oracle

        rng = np.random.default_rng(1000 + args.seed)
        tok = np.sort(rng.choice(s.T, min(args.cpu_tokens, s.T), replace=False))
        log(f"CPU oracle on {len(tok)} sampled tokens")
        t0 = time.perf_counter()
        oracle.layer_tokens(x_np, wr_np, bias_np, lambda e: canon[e], s.K, tok, fmt=s.fmt,
                            shared=(canon[s.E], wg_np) if s.shared else None)
        dt = time.perf_counter() - t0
        cpu = {"value": round(len(tok) / dt, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{len(tok)} random tokens of the {s.name} layer, full layer per token "
                         f"(router, top-K, quantize, {s.K + s.shared} expert FFNs, combine) in double; {dt:.2f} s"}

    line = {
        "metric": METRIC,
        "value": round(s.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": s.name, "T": s.T, "H": s.H, "E": s.E, "K": s.K, "I": s.I,
                   "weights": "2-bit codes, fp16 scale per 32, " + ("w = d(q-1)" if s.fmt == "q2_0" else "w = d(q-1.5)"),
                   "activations": "int8, fp32 scale per 32",
                   "router_matrix": "prepared per call" if args.router_per_call else "prepared once",
                   "shared_expert": bool(s.shared)},
        "kernel_ms": {k: round(v, 4) for k, v in kernel_ms.items()},
        "int8_ops_per_step": 2.0 * n * 3 * s.H * s.I,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
