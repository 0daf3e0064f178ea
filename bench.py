"""Benchmark of the IA layer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 1.3b|125m|1.3b_long|caduceus]
                    [--no-cpu] [--no-decode] [--no-backward]

A step is one causal (or, for the genomic workload, bidirectional) IA layer forward over the
whole synthetic batch, through ia_prefill_fwd: per-head tables, segment end states, carry
scan and the chunked MFMA pass with outputs.  Inputs are resident in HBM before timing starts.
Prints one JSON line: prefill tokens/s, the roofline position of the dominant kernel
(measured with HIP events around that kernel, over a timed loop), decode-step latency at
batch 1/16/64 (hipGraph-captured and eager), the backward pass of the same layer (its time and
its position against the fp32 vector peak), and the CPU oracle's throughput on a sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X
BF16_PEAK = 2.5e15         # dense bf16 MFMA FLOP/s, MI355X

WORKLOADS = {
    "1.3b": ("1.3B-shaped IA layer prefill", lambda W: W.l1p3b(), False),
    "125m": ("125M-shaped IA layer prefill", lambda W: W.l125m(), False),
    "1.3b_long": ("1.3B-shaped IA layer prefill, 3.5x length (N=7168)",
                  lambda W: W.l1p3b(N=7168), False),
    "caduceus": ("Caduceus-style bidirectional genomic IA layer", lambda W: W.caduceus(), True),
}


def alg_counts(B, N, H, F, D, M, in_bytes=2, out_bytes=2, chunk=64, dirs=1):
    """Algorithmic FLOPs and HBM bytes of one layer forward (chunked method at C=64):
    per token, head and direction 2[C(F+4M+D) + 4M(F+D)] FLOP; per token and head
    (2F+D) input bytes and D output bytes."""
    flops = 2.0 * (chunk * (F + 4 * M + D) + 4 * M * (F + D)) * B * N * H * dirs
    byts = float((2 * F + D) * in_bytes + D * out_bytes) * B * N * H
    return flops, byts


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(h)) == 0
            out.append(h.value)
        self.made += out
        return out

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.rt.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.rt.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a),
                                           ctypes.c_void_p(b)) == 0
        return f.value

    def close(self):
        for h in self.made:
            self.rt.hipEventDestroy(ctypes.c_void_p(h))


def bench_prefill(args, torch, ia, W):
    title, make, bidir = WORKLOADS[args.workload]
    inp = make(W)
    sh = inp["shape"]
    B, H, N, F, D, M = sh["B"], sh["H"], sh["N"], sh["F"], sh["D"], sh["M"]
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv")
    lam = torch.from_numpy(inp["lam"]).cuda()
    beta = torch.from_numpy(inp["beta"]).cuda()
    out_dtype = torch.bfloat16
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_BF16, 1e-6, bidir, 0)
    o = torch.empty((B, N, H, D), dtype=out_dtype, device="cuda")
    ws = torch.empty(max(ia.ia_prefill_workspace_bytes(desc), 16), dtype=torch.uint8,
                     device="cuda")

    def step():
        ia.ia_prefill_fwd(desc, q, k, v, lam, beta, None, o, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps

    # Per-kernel durations from HIP events around each launch, over a second timed loop.
    hev = HipEvents()
    max_l = 8
    evs = [hev.create(2 * max_l) for _ in range(args.steps)]
    kinds = None
    for s in range(args.steps):
        kinds = ia.ia_prefill_fwd_profiled(desc, q, k, v, lam, beta, None, o, ws, evs[s])
    torch.cuda.synchronize()
    per_kind = {}
    for s in range(args.steps):
        for i, kd in enumerate(kinds):
            per_kind.setdefault(ia.KIND_NAMES[kd], []).append(hev.ms(evs[s][2 * i],
                                                                     evs[s][2 * i + 1]))
    hev.close()
    kern_ms = {name: float(np.mean(v)) for name, v in per_kind.items()}

    dirs = 2 if bidir else 1
    flops, byts = alg_counts(B, N, H, F, D, M, dirs=dirs)
    dom = kern_ms["chunk"] * dirs            # the output pass (once per direction)
    roof = {"bound": "hbm", "achieved": byts / (dom * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9,
            "unit": "GB/s", "frac": byts / (dom * 1e-3) / HBM_PEAK,
            "traffic": None if bidir else profiled_traffic(args.workload),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, scaled)",
            "alg_bytes_per_launch": byts / dirs,
            "kernel": "chunk_prefill_kernel (output pass)"}
    mfma = {"achieved": flops / (dom * 1e-3) / 1e12, "peak": BF16_PEAK / 1e12,
            "unit": "TFLOP/s", "frac": flops / (dom * 1e-3) / BF16_PEAK,
            "whole_step_frac": flops / (ms * 1e-3) / BF16_PEAK}
    cfg = {"workload": title, "B": B, "H": H, "N": N, "F": F, "Dv": D, "M": M,
           "chunk": 64, "in_dtype": "bf16", "out_dtype": "bf16",
           "bidirectional": bidir}
    return dict(ms=ms, tokens=B * N, cfg=cfg, roofline=roof, mfma=mfma, kernels_ms=kern_ms,
                inp=inp)


KERNEL_SOURCES = ["ssm_sequence_mixer_amd/csrc/ia_chunk.hpp",
                  "ssm_sequence_mixer_amd/csrc/ia_device.hpp",
                  "ssm_sequence_mixer_amd/csrc/ia_kernels.hpp"]
TRAFFIC_PROFILE = {"1.3b": "profiles/chunk_prefill_1p3b_traffic.md"}


def profiled_traffic(workload):
    """HBM bytes per launch of the output pass from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (counters scaled by a streaming kernel of known size), or None when
    there is none for this workload or the kernel sources changed since it was taken."""
    import hashlib
    path = TRAFFIC_PROFILE.get(workload)
    if path is None or not os.path.exists(os.path.join(ROOT, path)):
        return None
    fields = {}
    for line in open(os.path.join(ROOT, path)):
        if ":" in line and line.strip().split(":")[0] in ("traffic_bytes_per_launch",
                                                          "kernel_sources_sha256"):
            key, val = line.strip().split(":", 1)
            fields[key] = val.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"])


def bench_decode(torch, ia, W, batches=(1, 16, 64), steps=256):
    res = {}
    for Bd in batches:
        wl = W.decode(Bd, steps=steps, prefix=32)
        sh = wl["shape"]
        H, F, D, M = sh["H"], sh["F"], sh["D"], sh["M"]
        lam = torch.from_numpy(wl["lam"]).cuda()
        beta = torch.from_numpy(wl["beta"]).cuda()
        pre = {n: torch.from_numpy(wl["prefix"][n]).to(torch.bfloat16).cuda() for n in "qkv"}
        stp = {n: torch.from_numpy(wl["steps"][n]).to(torch.bfloat16).cuda() for n in "qkv"}
        st = ia.new_state(Bd, H, M, F, D)
        ia.prefill(pre["q"], pre["k"], pre["v"], lam, beta, state=st, want_output=False)
        o = torch.empty((steps, Bd, H, D), dtype=torch.float32, device="cuda")
        desc = ia.make_desc(Bd, H, 1, F, D, M, ia.IA_BF16, ia.IA_F32)

        def run_all():
            for t in range(steps):
                ia.ia_decode_step(desc, stp["q"][t], stp["k"][t], stp["v"][t], lam, beta, st,
                                  o[t])

        run_all()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_all()
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) / steps * 1e3
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                run_all()
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) / steps * 1e3
        step_bytes = Bd * H * (16 * M * (F + D + 1) + (2 * F + D) * 2 + D * 4)
        res[f"B{Bd}"] = {"graph_us_per_step": graph_us, "eager_us_per_step": eager_us,
                         "tokens_per_s": Bd / (graph_us * 1e-6),
                         "hbm_frac": step_bytes / (graph_us * 1e-6) / HBM_PEAK,
                         "bytes_per_step": step_bytes}
        del g
        if Bd == 16:
            # the same steps with a readout matrix R per head (the M^2 term of a decode step)
            rng = np.random.default_rng(7)
            R = (np.eye(M) + 0.1 * rng.standard_normal((H, M, M))).astype(np.complex64)
            Rd = torch.from_numpy(R).cuda()
            for _ in range(2):
                for t in range(steps):
                    ia.ia_decode_step_readout(desc, stp["q"][t], stp["k"][t], stp["v"][t], lam,
                                              beta, Rd, st, o[t])
                torch.cuda.synchronize()
            e0.record()
            for t in range(steps):
                ia.ia_decode_step_readout(desc, stp["q"][t], stp["k"][t], stp["v"][t], lam, beta,
                                          Rd, st, o[t])
            e1.record()
            torch.cuda.synchronize()
            res[f"B{Bd}"]["readout_matrix_eager_us_per_step"] = e0.elapsed_time(e1) / steps * 1e3
    return res


FP32_PEAK = 157.3e12        # fp32 vector FLOP/s, MI355X


def bwd_alg_flops(B, N, H, F, D, M):
    """Algorithmic FLOPs of the backward pass (fp32 VALU): per token, head and mode, the state
    recompute 14 (F + D) and the reverse sweep 44 F + 41 D (a complex multiply counted 6, a
    complex-by-real multiply-add 4)."""
    return float(14 * (F + D) + 44 * F + 41 * D) * M * B * N * H


def bench_backward(torch, ia, inp, bidir=False, steps=5, warmup=2):
    """ia_prefill_bwd over the prefill workload (bf16 q, k, v; fp32 dO), from a zero state
    (both directions for the bidirectional workload)."""
    sh = inp["shape"]
    B, H, N, F, D, M = sh["B"], sh["H"], sh["N"], sh["F"], sh["D"], sh["M"]
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv")
    lam = torch.from_numpy(inp["lam"]).cuda()
    beta = torch.from_numpy(inp["beta"]).cuda()
    g = torch.Generator(device="cpu").manual_seed(550)
    dO = torch.randn((B, N, H, D), generator=g, dtype=torch.float32).cuda()
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_F32, bidir=bidir)
    ws = torch.empty(ia.ia_prefill_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    if N > 16384:   # the long genomic sequence: one timed step (a step takes seconds' share)
        steps, warmup = 1, 1
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dl = torch.empty((H, M), dtype=torch.complex64, device="cuda")
    db = torch.empty_like(dl)

    def step():
        ia.ia_prefill_bwd(desc, q, k, v, lam, beta, None, dO, dq, dk, dv, dl, db, None, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    fl = bwd_alg_flops(B, N, H, F, D, M) * (2 if bidir else 1)
    return {"us_per_step": us, "tokens_per_s": B * N / (us * 1e-6), "steps": steps,
            "dtype": "bf16 in, fp32 state and arithmetic", "workspace_bytes": ws.numel(),
            "alu": {"bound": "alu", "achieved": fl / (us * 1e-6) / 1e12,
                    "peak": FP32_PEAK / 1e12, "unit": "TFLOP/s",
                    "frac": fl / (us * 1e-6) / FP32_PEAK, "alg_flops": fl}}


def cpu_baseline(inp, bidir, budget_s=12.0):
    """The oracle as it stands, on the host cores, over a bounded sample of (b,h) slices."""
    import oracle
    cores = min(len(os.sched_getaffinity(0)), 16)
    sh = inp["shape"]
    B, H, N = sh["B"], sh["H"], sh["N"]
    slices = [(b, h) for b in range(B) for h in range(H)]
    # time one slice, then size the sample to about budget_s of wall time
    t = time.perf_counter()
    if bidir:
        oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], slices=slices[:1])
    else:
        oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], slices=slices[:1])
    one = time.perf_counter() - t
    n = int(max(1, min(len(slices), budget_s * cores / max(one, 1e-6))))
    n = max(cores, (n // cores) * cores) if n >= cores else n
    n = min(n, len(slices))
    sample = slices[:n]
    t = time.perf_counter()
    if bidir:
        oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], slices=sample,
                     threads=cores)
    else:
        oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], slices=sample,
                       threads=cores)
    wall = time.perf_counter() - t
    # layer tokens/s: B*N tokens need all B*H slices; the sample holds n of them
    value = (N * len(sample) / H) / wall
    return {"value": value, "unit": "tokens/s", "cores": min(cores, len(sample)),
            "kind": "oracle",
            "sample": f"{len(sample)} of {B * H} (b,h) slices x {N} tokens"
                      f"{' x 2 directions' if bidir else ''}, fp64 serial recurrence per "
                      f"slice, slices spread over {min(cores, len(sample))} threads; "
                      f"{wall:.1f} s wall; one slice alone {one:.2f} s"}


def calib_copy(torch, mib=256):
    """A plain elementwise kernel (negation, fp32) that reads and writes `mib` MiB once each:
    the reference point for FETCH_SIZE / WRITE_SIZE."""
    src = torch.ones(mib * 2 ** 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1.3b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain streaming kernel over 256 MiB (read 256 MiB, write "
                         "256 MiB) whose counter readings scale the hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer shards by (b,h) with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch

    import ia_workloads as W
    import ssm_sequence_mixer_amd as ia

    torch.cuda.init()
    if args.calib_copy:
        calib_copy(torch)
    pf = bench_prefill(args, torch, ia, W)
    dec = None if args.no_decode else bench_decode(torch, ia, W)
    bwd = None
    if not args.no_backward:
        bwd = bench_backward(torch, ia, pf["inp"], bidir=pf["cfg"]["bidirectional"])
    cpu = None if args.no_cpu else cpu_baseline(pf["inp"], pf["cfg"]["bidirectional"])
    line = {
        "metric": "IA layer fwd tokens/s (prefill) + decode step latency; % of MFMA/HBM roofline",
        "value": pf["tokens"] / (pf["ms"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": pf["cfg"],
        "roofline": pf["roofline"],
        "mfma": pf["mfma"],
        "kernels_ms": pf["kernels_ms"],
        "decode": dec,
        "backward": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
