#!/usr/bin/env python3
"""Benchmark of the routed-expert prompt MoE layer on one MI355X.

A step is one strata_moe_prefill call -- router, top-K, grouping, int8
quantization, gate/up + SwiGLU + int8 H, down + the weighted combine -- over a
chunk of T tokens whose inputs, packed experts and prepared router matrix
(strata_moe_prepare_router, once, like the packing; --router-per-call prepares
it inside every step instead) are already resident in HBM.  Default workload:
T = 8192, H = 2560, E = 512 experts, top-10, expert FFN I = 1024, seeded
synthetic inputs (the pages' own prompts and trained pack are not available).
The same run also times the 1024-token chunk (the weight-streaming end) on the
same experts and reports it in the same JSON line.

Prints one JSON line on stdout (progress goes to stderr):
  value        tokens/s of the layer over the timed steps (one GPU)
  layer        whole-layer int8-equivalent TOPS against the int8 and fp16
               MFMA peaks, median / min / cold-cache step times
  roofline     the dominant kernel's achieved rate against the int8 peak
               (its fp16 fraction beside it), measured with HIP events on the
               launch stream over the timed steps
  stream_all_1k  the 1024-token chunk: ms per step, the hit experts' weight
               bytes per second against the 8 TB/s HBM peak
  streamed     the same layer with every expert streamed from pinned host
               memory through rings of 96, 384 and 512 device slots
  small_t      32- to 256-token chunks: ms per step, gate/up's weight GB/s,
               for the layer's own kernel choice ("default") and each forced
               one (MFMA only, the GEMV, the GEMV on per-slot q8_1 inputs)
  mfma_measured  the matrix unit's rates measured on this device
  hbm_measured the read bandwidth a plain streaming kernel gets on this
               device (the achievable ceiling beside the published 8 TB/s)
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
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE prefill layer tokens/s at T=8192 (512 exp, top-10); % int8 MFMA / HBM peak"
PEAK_I8_TOPS = 5000.0     # MI355X dense int8 MFMA (5.0 POPS)
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
SECOND = "stream_all_1k"  # the weight-streaming chunk reported beside the headline


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
    ap.add_argument("--second-steps", type=int, default=200,
                    help="timed steps of the 1024-token chunk (0 = skip it)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="steps timed after a 512 MiB scrub each (cold Infinity Cache; 0 = skip)")
    ap.add_argument("--no-probe", action="store_true", help="skip the matrix-unit rate measurements")
    ap.add_argument("--rings", default="96,384,512",
                    help="ring sizes (slots) of the streamed-experts measurement, comma separated ('' = skip)")
    ap.add_argument("--ring-steps", type=int, default=5, help="timed steps per ring size")
    ap.add_argument("--small-t", default="window_32,window_64,window_128,short_256",
                    help="small-T workloads timed on the same experts, comma separated ('' = skip)")
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


def time_steps(qm, torch, s, x, wr, experts, out, steps: int, warmup: int, scrub=None):
    """Runs warmup + steps layer calls; returns (ms per step over the whole
    timed region, per-step ms list, per-kernel mean ms).  With scrub (a
    device tensor), each timed step is preceded by a write of it (outside the
    step's events), so the step starts with a cold Infinity Cache."""
    for _ in range(warmup):
        qm.strata_moe_prefill(x, wr, experts, s.K, out)
    torch.cuda.synchronize()
    qm.strata_moe_timing(True, steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if scrub is not None:
            scrub.fill_(float(i))
        evs[i][0].record()
        qm.strata_moe_prefill(x, wr, experts, s.K, out)
        evs[i][1].record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    kt = qm.strata_moe_timing_read()
    qm.strata_moe_timing(False)
    kernel_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in kt.items()}
    return per, kernel_ms


def region_ms(qm, torch, s, x, wr, experts, out, steps: int):
    """ms per step over one timed region of back-to-back steps, bracketed by
    synchronisation and two events (the contract's timing)."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        qm.strata_moe_prefill(x, wr, experts, s.K, out)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, 1e3 * (time.perf_counter() - wall0) / steps


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "" where it cannot be read."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def hit_experts(torch, ids, nexp: int) -> int:
    return int((torch.bincount(ids.reshape(-1).long(), minlength=nexp) > 0).sum())


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
    base_experts = experts
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

    # the contract's timed region: K back-to-back steps between two events
    log(f"timing {args.steps} steps")
    ms_per_step, wall_ms = region_ms(qm, torch, s, x, wr, experts, out, args.steps)
    # the same steps again with events around every step and every kernel
    per, kernel_ms = time_steps(qm, torch, s, x, wr, experts, out, args.steps, 0)
    log(f"{ms_per_step:.3f} ms/step (wall {wall_ms:.3f}); per step median {statistics.median(per):.3f}, "
        f"min {min(per):.3f}; per kernel " + ", ".join(f"{k} {v:.3f}" for k, v in kernel_ms.items()))
    cold = None
    if args.cold_steps > 0:
        scrub = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        per_cold, _ = time_steps(qm, torch, s, x, wr, experts, out, args.cold_steps, 0, scrub=scrub)
        cold = statistics.median(per_cold)
        del scrub
        log(f"cold Infinity Cache: median {cold:.3f} ms/step over {args.cold_steps} steps")
    qm.strata_moe_set_workspace(None)

    if args.copy_probe_mib:
        a = torch.empty((args.copy_probe_mib << 20) // 4, dtype=torch.float32, device=dev).uniform_()
        b = torch.empty_like(a)
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        flush.fill_(1.0)  # 512 MiB written: evicts the 256 MiB Infinity Cache
        torch.cuda.synchronize()
        torch.neg(a, out=b)  # reads and writes copy_probe_mib MiB
        torch.cuda.synchronize()
        del flush, a, b
        log(f"copy probe: {args.copy_probe_mib} MiB")

    n = s.T * (s.K + s.shared)  # grouped rows: K routed pairs per token, plus the shared expert's
    ops = {"gate_up": 2.0 * n * 2 * s.I * s.H, "down": 2.0 * n * s.H * s.I}
    layer_ops = 2.0 * n * 3 * s.H * s.I
    expert_bytes = 3 * s.H * s.I * (2 / 8 + 2 / 32)  # packed gate, up and down of one expert
    dominant = max(kernel_ms, key=kernel_ms.get)
    traffic = measured_traffic(dominant, s.name) if dominant in ops else None
    if dominant in ops and n / s.E >= 64:
        # many rows per expert: the grouped GEMM is a dense contraction
        achieved = ops[dominant] / (kernel_ms[dominant] * 1e-3) / 1e12
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_I8_TOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_I8_TOPS, 4), "traffic": traffic,
                    "peak_f16": PEAK_F16_TFLOPS, "frac_f16": round(achieved / PEAK_F16_TFLOPS, 4)}
    elif dominant in ops:
        # few rows per expert: the GEMM streams the hit experts' packed weights once
        hit = hit_experts(torch, dbg_ids, s.E + s.shared)
        share = (2 / 3) if dominant == "gate_up" else (1 / 3)
        achieved = hit * expert_bytes * share / (kernel_ms[dominant] * 1e-3) / 1e9
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": None, "traffic": None}
    layer_tops = layer_ops / (ms_per_step * 1e-3) / 1e12
    layer = {"int8_ops_per_step": layer_ops, "tops": round(layer_tops, 2),
             "frac_int8": round(layer_tops / PEAK_I8_TOPS, 4), "frac_f16": round(layer_tops / PEAK_F16_TFLOPS, 4),
             "median_ms": round(statistics.median(per), 4), "min_ms": round(min(per), 4),
             "cold_ms": None if cold is None else round(cold, 4),
             "hit_experts": hit_experts(torch, dbg_ids, s.E + s.shared)}

    second = None
    if args.second_steps > 0 and s.name != SECOND:
        s2 = S.shape(SECOND)
        if (s2.E, s2.H, s2.I, s2.fmt) == (s.E, s.H, s.I, s.fmt) and not s.shared and not s.skewed:
            x2 = torch.from_numpy(S.activations(s2, args.seed)).to(dev)
            ex2 = base_experts if args.router_per_call else base_experts.with_prepared_router(wr)
            out2 = torch.empty_like(x2)
            ms2, _ = region_ms(qm, torch, s2, x2, wr, ex2, out2, 10)  # warm
            ms2, _ = region_ms(qm, torch, s2, x2, wr, ex2, out2, args.second_steps)
            per2, kms2 = time_steps(qm, torch, s2, x2, wr, ex2, out2, min(args.second_steps, 100), 0)
            ids2 = qm.strata_moe_prefill_debug(x2, wr, ex2, s2.K, out2)["ids"]
            torch.cuda.synchronize()
            hit2 = hit_experts(torch, ids2, s2.E)
            wbytes = hit2 * expert_bytes
            second = {"workload": s2.name, "T": s2.T, "ms_per_step": round(ms2, 4),
                      "median_ms": round(statistics.median(per2), 4), "min_ms": round(min(per2), 4),
                      "tokens_per_s": round(s2.T / (ms2 * 1e-3), 1), "hit_experts": hit2,
                      "weight_bytes": wbytes, "weight_gbs": round(wbytes / (ms2 * 1e-3) / 1e9, 1),
                      "frac_hbm": round(wbytes / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "kernel_ms": {k: round(v, 4) for k, v in kms2.items()}}
            log(f"{s2.name}: {ms2:.3f} ms/step, hit experts' weights at {second['weight_gbs']} GB/s "
                f"({100 * second['frac_hbm']:.1f}% of 8 TB/s)")

    small_t = None
    names = [w for w in args.small_t.split(",") if w.strip()]
    if names and not s.shared and not s.skewed:
        small_t = {}
        gu_bytes = 2 * s.I * s.H * (2 / 8 + 2 / 32)  # one expert's packed gate/up matrix
        for name in names:
            s3 = S.shape(name)
            if (s3.E, s3.H, s3.I, s3.fmt) != (s.E, s.H, s.I, s.fmt):
                continue
            x3 = torch.from_numpy(S.activations(s3, args.seed)).to(dev)
            ex3 = base_experts if args.router_per_call else base_experts.with_prepared_router(wr)
            out3 = torch.empty_like(x3)
            ids3 = qm.strata_moe_prefill_debug(x3, wr, ex3, s3.K, out3)["ids"]
            hit3 = hit_experts(torch, ids3, s3.E)
            entry = {"T": s3.T, "hit_experts": hit3}
            arms = (("default", 0), ("mfma_only", qm.FLAG_NO_GEMV), ("gemv", qm.FLAG_GEMV_ALWAYS),
                    ("gemv_per_slot_q8", qm.FLAG_GEMV_ALWAYS | qm.FLAG_PER_SLOT_Q8))
            for label, flags in arms:
                exf = ex3.with_flags(flags)
                region_ms(qm, torch, s3, x3, wr, exf, out3, 20)  # warm
                ms3, _ = region_ms(qm, torch, s3, x3, wr, exf, out3, 200)
                per3, kms3 = time_steps(qm, torch, s3, x3, wr, exf, out3, 100, 0)
                gbs = hit3 * gu_bytes / (kms3["gate_up"] * 1e-3) / 1e9
                entry[label] = {"ms_per_step": round(ms3, 4), "median_ms": round(statistics.median(per3), 4),
                                "gate_up_ms": round(kms3["gate_up"], 4), "down_ms": round(kms3["down"], 4),
                                "gate_up_weight_gbs": round(gbs, 1), "gate_up_frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
                log(f"{name} [{label}]: {ms3:.3f} ms/step, gate/up {kms3['gate_up']:.4f} ms "
                    f"({gbs:.0f} GB/s of hit experts' weights), down {kms3['down']:.4f} ms")
            small_t[name] = entry

    streamed = None
    rings = [int(r) for r in args.rings.split(",") if r.strip()]
    if rings and not s.shared:
        # the same experts in pinned host memory, expert e's gate/up and down blobs
        # side by side (one DMA each), copied from the resident blobs
        host = qm.HostExperts(s.E, s.H, s.I, fmt=s.fmt)
        hv = host.host.view(s.E, host.slot_bytes)
        hv[:, :host.gate_up_bytes].copy_(base_experts.gate_up.view(s.E, -1)[:, :host.gate_up_bytes])
        hv[:, host.gate_up_bytes:].copy_(base_experts.down.view(s.E, -1)[:, :host.slot_bytes - host.gate_up_bytes])
        host = host.with_router_bias(bias)
        if not args.router_per_call:
            host = host.with_prepared_router(wr)
        y_res = qm.strata_moe_prefill(x, wr, experts, s.K, torch.empty_like(x))
        streamed = {"bytes_per_step": s.E * host.slot_bytes, "ms_per_step": {}, "host_to_device_gbs": {},
                    "bitwise_equal_to_resident": True}
        for R in rings:
            ring = qm.Ring(R, s.H, s.I, device=dev)
            ys = torch.empty_like(x)
            for _ in range(2):
                qm.strata_moe_prefill_streamed(x, wr, host, ring, s.K, ys)
            torch.cuda.synchronize()
            streamed["bitwise_equal_to_resident"] &= bool(torch.equal(ys, y_res))
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for _ in range(args.ring_steps):
                qm.strata_moe_prefill_streamed(x, wr, host, ring, s.K, ys)
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / args.ring_steps
            ring.close()
            streamed["ms_per_step"][str(R)] = round(ms, 3)
            streamed["host_to_device_gbs"][str(R)] = round(streamed["bytes_per_step"] / (ms * 1e-3) / 1e9, 1)
            log(f"streamed experts, ring of {R} slots: {ms:.3f} ms/step "
                f"({streamed['host_to_device_gbs'][str(R)]} GB/s of expert blobs over the host link)")
        del host

    mfma = hbm = None
    if not args.no_probe:
        from quantized_routed_expert_logits_amd import probe

        mfma = {}
        for kind in probe.KINDS:
            rate, _ = probe.strata_probe_mfma_rate(kind)
            mfma[kind] = round(rate / 1e12, 1)
        f16_blocks, _ = probe.strata_probe_scaled_blocks(False)
        i8_blocks, _ = probe.strata_probe_scaled_blocks(True)
        mfma["unit"] = "TOP/s (2 M N K per MFMA, 8 chains per wave, all SIMDs)"
        mfma["scaled_blocks_f16"] = round(f16_blocks / 1e12, 3)
        mfma["scaled_blocks_i8"] = round(i8_blocks / 1e12, 3)
        mfma["scaled_blocks_unit"] = "T output-blocks/s (32-wide block products, each scaled into fp32)"
        # the same fp16 form at the gate/up kernel's shape (6 tiles of 32 x 32 per wave and block), and with
        # the 32x32x16 MFMA: the ceiling of the exact block-scaled products, operands in registers
        for form in ("16x16x32", "32x32x16"):
            mfma[f"scaled_tiles6_f16_{form}"] = round(probe.strata_probe_scaled_tiles(form, 6)[0] / 1e12, 3)
        # that shape with activation loads (0), plus the unpack and the LDS exchange, a barrier per block
        # (1) or per two blocks (2)
        for step in (0, 1, 2):
            mfma[f"block_step{step}"] = round(probe.strata_probe_block_step(step)[0] / 1e12, 3)
        log("MFMA rates (TOP/s): " + ", ".join(f"{k} {mfma[k]}" for k in probe.KINDS)
            + f"; scaled blocks fp16 {mfma['scaled_blocks_f16']} vs int8 {mfma['scaled_blocks_i8']} T/s"
            + f"; at the kernel's 6 tiles: 16x16x32 {mfma['scaled_tiles6_f16_16x16x32']}, "
            + f"32x32x16 {mfma['scaled_tiles6_f16_32x32x16']} T/s; block step "
            + ", ".join(str(mfma[f"block_step{i}"]) for i in range(3)) + " T/s")
        reads = {str(g): round(probe.strata_probe_hbm_read(2 << 30, g)[0], 1) for g in (1024, 4096, 16384)}
        hbm = {"read_gbs": max(reads.values()), "by_workgroups": reads, "bytes": 2 << 30,
               "kernel": "16-byte loads, 4 in flight per thread, grid-stride, 256 threads per workgroup"}
        log(f"HBM streaming read: {hbm['read_gbs']} GB/s (by workgroups {reads})")

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
                         f"(router, top-K, quantize, {s.K + s.shared} expert FFNs, combine) in double; {dt:.2f} s",
               "cpu_model": cpu_model()}

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
        "int8_ops_per_step": layer_ops,
        "layer": layer,
        "roofline": roofline,
        "stream_all_1k": second,
        "streamed": streamed,
        "small_t": small_t,
        "mfma_measured": mfma,
        "hbm_measured": hbm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
