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

    if args.warmup is None:
        # Untimed steps until the GPU has run the workload for half a second: the clocks ramp
        # up over the first ~100 ms of load, and a short warmup times the ramp, not the kernels.
        args.warmup = 0
        t_start = time.perf_counter()
        while args.warmup < 3 or time.perf_counter() - t_start < 0.5:
            for _ in range(10):
                step()
            args.warmup += 10
            torch.cuda.synchronize()
    else:
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
            "scope": "dominant kernel only: the output pass's algorithmic bytes over its own "
                     "mean launch time (HIP events on its stream)",
            "kernel": "chunk_prefill_kernel (output pass)",
            "kernel_us": dom * 1e3 / dirs}
    mfma = {"scope": "dominant kernel only", "achieved": flops / (dom * 1e-3) / 1e12,
            "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s", "frac": flops / (dom * 1e-3) / BF16_PEAK}
    whole = {"scope": "whole step (every launch of ia_prefill_fwd), ms_per_step",
             "hbm_achieved_GBps": byts / (ms * 1e-3) / 1e9,
             "hbm_frac": byts / (ms * 1e-3) / HBM_PEAK,
             "mfma_achieved_TFLOPs": flops / (ms * 1e-3) / 1e12,
             "mfma_frac": flops / (ms * 1e-3) / BF16_PEAK}
    # The readout-matrix variant (a R in place of a, R a per-head M x M complex matrix) on the
    # same inputs, timed the same way; chunk 32 where its 64-token LDS layout has no room.
    rng = np.random.default_rng(7)
    R = np.eye(M)[None] + 0.05 * (rng.standard_normal((H, M, M)) +
                                  1j * rng.standard_normal((H, M, M))) / np.sqrt(M)
    Rd = torch.from_numpy(R.astype(np.complex64)).cuda()
    ws_r = torch.empty(max(ia.ia_prefill_readout_workspace_bytes(desc), 16), dtype=torch.uint8,
                       device="cuda")

    def step_r():
        ia.ia_prefill_fwd_readout(desc, q, k, v, lam, beta, Rd, None, o, ws_r)

    for _ in range(args.warmup):
        step_r()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step_r()
    t1.record()
    torch.cuda.synchronize()
    ms_r = t0.elapsed_time(t1) / args.steps
    readout = {"scope": "ia_prefill_fwd_readout on the same inputs, ms_per_step",
               "ms_per_step": ms_r, "vs_plain": ms_r / ms,
               "chunk": 32 if (F == 128 and D == 128 and M == 64) else 64}

    cfg = {"workload": title, "B": B, "H": H, "N": N, "F": F, "Dv": D, "M": M,
           "chunk": 64, "in_dtype": "bf16", "out_dtype": "bf16",
           "bidirectional": bidir}
    return dict(ms=ms, tokens=B * N, cfg=cfg, roofline=roof, mfma=mfma, whole=whole,
                kernels_ms=kern_ms, inp=inp, readout=readout)


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


MALL_BYTES = 256 * 2 ** 20   # MI355X Infinity Cache


def _graph_us(torch, run, reps=1):
    """Per-call time of run() captured in one hipGraph (run enqueues `reps` steps)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / reps


def bench_decode(torch, ia, W, batches=(1, 16, 64), steps=256):
    """Decode-step latency after a 32-token chunked prefill, 256 steps, eager and graph-
    captured.  "hot": one state, resident in the MALL between steps at these sizes; "cold":
    the same steps rotating over enough copies of the state that their total exceeds the
    MALL, so every step reads its state from HBM.  "prefix_16k": graph latency after a
    16,384-token prefix instead (the step's work does not depend on the prefix)."""
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
        qs = [stp["q"][t] for t in range(steps)]
        ks = [stp["k"][t] for t in range(steps)]
        vs = [stp["v"][t] for t in range(steps)]

        def run_all(states=(st,)):
            for t in range(steps):
                ia.ia_decode_step(desc, qs[t], ks[t], vs[t], lam, beta,
                                  states[t % len(states)], o[t])

        run_all()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_all()
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) / steps * 1e3
        graph_us = _graph_us(torch, run_all, steps)
        state_bytes = Bd * H * 8 * M * (F + D + 1)
        step_bytes = Bd * H * (16 * M * (F + D + 1) + (2 * F + D) * 2 + D * 4)
        # cold: copies of the state whose total exceeds the MALL
        n_sets = max(2, -(-2 * MALL_BYTES // state_bytes))
        sets = [tuple(x.clone() for x in st) for _ in range(n_sets)]
        cold_us = _graph_us(torch, lambda: run_all(sets), steps)
        del sets
        r = {"graph_us_per_step": graph_us, "eager_us_per_step": eager_us,
             "tokens_per_s": Bd / (graph_us * 1e-6),
             "hbm_frac_hot": step_bytes / (graph_us * 1e-6) / HBM_PEAK,
             "cold_graph_us_per_step": cold_us,
             "hbm_frac_cold": step_bytes / (cold_us * 1e-6) / HBM_PEAK,
             "cold_state_sets": n_sets, "bytes_per_step": step_bytes,
             "state_bytes": state_bytes}
        if Bd in (1, 16):
            # prefix flatness: the state after 16,384 tokens (state-only chunked prefill)
            rng = np.random.default_rng([55, Bd])
            long = {n: torch.from_numpy(W.round_bf16(
                rng.standard_normal((Bd, 16384, H, F if n != "v" else D), dtype=np.float32)
                / np.sqrt(F))).to(torch.bfloat16).cuda() for n in "qkv"}
            st_long = ia.new_state(Bd, H, M, F, D)
            ia.prefill(long["q"], long["k"], long["v"], lam, beta, state=st_long,
                       want_output=False)
            del long
            long_us = _graph_us(torch, lambda: run_all((st_long,)), steps)
            r["prefix_16k_graph_us_per_step"] = long_us
            r["prefix_16k_over_32"] = long_us / graph_us
        if Bd == 16:
            # the same steps with a readout matrix R per head (the M^2 term of a decode step)
            rng = np.random.default_rng(7)
            R = (np.eye(M) + 0.1 * rng.standard_normal((H, M, M))).astype(np.complex64)
            Rd = torch.from_numpy(R).cuda()
            for _ in range(2):
                for t in range(steps):
                    ia.ia_decode_step_readout(desc, qs[t], ks[t], vs[t], lam, beta, Rd, st, o[t])
                torch.cuda.synchronize()
            e0.record()
            for t in range(steps):
                ia.ia_decode_step_readout(desc, qs[t], ks[t], vs[t], lam, beta, Rd, st, o[t])
            e1.record()
            torch.cuda.synchronize()
            r["readout_matrix_eager_us_per_step"] = e0.elapsed_time(e1) / steps * 1e3
        res[f"B{Bd}"] = r
    return res


def bench_block(torch, ia, W, inp, layers=24, reps=20):
    """The block's edges on the prefill workload (ia_block_prologue with a 4-tap convolution,
    RoPE and the normalisation; ia_block_gate on o), and a graph-captured decode of a stack of
    `layers` blocks at batch 1 (per layer: prologue of one token, ia_decode_step with identity
    features, gate), the 1.3B-shaped layer's sizes."""
    sh = inp["shape"]
    B, H, N, F, D, M = sh["B"], sh["H"], sh["N"], sh["F"], sh["D"], sh["M"]
    tb = torch.bfloat16
    q, k, v = (torch.from_numpy(inp[n]).to(tb).cuda() for n in "qkv")
    rng = np.random.default_rng(11)
    conv = tuple(torch.from_numpy((rng.standard_normal((H, C, 4)) * 0.4).astype(np.float32)).cuda()
                 for C in (F, F, D))
    norm = (torch.ones((H, F + D), device="cuda"), torch.zeros((H, F + D), device="cuda"))
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_BF16)
    p = ia.block_params(conv, 1e4, 0, norm)
    fq, fk, vo = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    g = torch.randn((B, N, H, D), device="cuda").to(tb)
    o = torch.randn((B, N, H, D), device="cuda").to(tb)
    out = torch.empty_like(o)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    pro_us = timed(lambda: ia.ia_block_prologue(desc, p, q, k, v, None, None, fq, fk, vo))
    gate_us = timed(lambda: ia.ia_block_gate(desc, o, g, out))
    pro_bytes = 2.0 * B * N * H * (2 * F + D) * 2
    gate_bytes = 3.0 * B * N * H * D * 2
    res = {"scope": "1.3B-shaped prefill workload, bf16",
           "prologue_us": pro_us, "prologue_hbm_frac": pro_bytes / (pro_us * 1e-6) / HBM_PEAK,
           "gate_us": gate_us, "gate_hbm_frac": gate_bytes / (gate_us * 1e-6) / HBM_PEAK}

    # stack decode, batch 1: `layers` blocks with their own states, two tokens per replay (the
    # convolution state alternates between two buffers)
    Bd = 1
    wl = W.decode(Bd, steps=2, prefix=32)
    lam = torch.from_numpy(wl["lam"]).cuda()
    beta = torch.from_numpy(wl["beta"]).cuda()
    dd = ia.make_desc(Bd, H, 1, F, D, M, ia.IA_BF16, ia.IA_BF16, identity_features=True)
    d1 = ia.make_desc(Bd, H, 1, F, D, M, ia.IA_BF16, ia.IA_BF16)
    xs = [tuple(torch.randn((Bd, 1, H, C), device="cuda").to(tb) for C in (F, F, D))
          for _ in range(2)]
    gts = [torch.randn((Bd, 1, H, D), device="cuda").to(tb) for _ in range(2)]
    L = []
    for _ in range(layers):
        st = ia.new_state(Bd, H, M, F, D)
        cs = [torch.zeros((Bd, H, 3, 2 * F + D), device="cuda") for _ in range(2)]
        feats = tuple(torch.empty((Bd, 1, H, C), device="cuda", dtype=tb) for C in (F, F, D))
        ot = torch.empty((Bd, 1, H, D), device="cuda", dtype=tb)
        L.append((st, cs, feats, ot))
    ps = [ia.block_params(conv, 1e4, pos, norm) for pos in (32, 33)]

    def run_stack():
        for t in range(2):
            x, gt = xs[t], gts[t]
            for st, cs, feats, ot in L:
                ia.ia_block_prologue(d1, ps[t], x[0], x[1], x[2], cs[t], cs[1 - t], *feats)
                ia.ia_decode_step(dd, feats[0][:, 0], feats[1][:, 0], feats[2][:, 0], lam, beta,
                                  st, ot[:, 0])
                ia.ia_block_gate(d1, ot, gt, ot)
    def run_stack_fused():
        for t in range(2):
            x, gt = xs[t], gts[t]
            for st, cs, feats, ot in L:
                ia.ia_block_decode_step(d1, ps[t], x[0][:, 0], x[1][:, 0], x[2][:, 0], cs[t],
                                        cs[1 - t], gt[:, 0], lam, beta, st, ot[:, 0])
    run_stack()
    run_stack_fused()
    torch.cuda.synchronize()
    stack_us = _graph_us(torch, run_stack, 2)
    fused_us = _graph_us(torch, run_stack_fused, 2)
    res.update({"stack_layers": layers, "stack_batch": Bd,
                "stack_graph_us_per_token": stack_us,
                "stack_graph_us_per_layer": stack_us / layers,
                "stack_scope": "per layer: prologue (conv state, RoPE, norm) of one token, "
                               "ia_decode_step with identity features, gate; one hipGraph",
                "stack_fused_graph_us_per_token": fused_us,
                "stack_fused_graph_us_per_layer": fused_us / layers,
                "stack_fused_scope": "the same with one ia_block_decode_step per layer"})
    return res


FP32_PEAK = 157.3e12        # fp32 vector FLOP/s, MI355X


def bench_gated(torch, ia, inp, plain_ms=None, reps=20):
    """Selective writing and memory decay (ia_prefill_fwd_gated: bf16 inputs on the chunked
    MFMA prefill with the gates folded into each chunk) on the prefill workload's q, k, v, with
    write gates in [0.5, 1) and decay gates in [0.9, 1), bf16 output: per-step time, tokens/s,
    the ratio to the ungated step, and the fractions of the bf16 MFMA peak (the ungated layer's
    algorithmic FLOPs: the gates add element-wise work only) and of HBM (the ungated bytes
    plus the two fp32 gates per token and head)."""
    sh = inp["shape"]
    B, H, N, F, D, M = sh["B"], sh["H"], sh["N"], sh["F"], sh["D"], sh["M"]
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv")
    lam = torch.from_numpy(inp["lam"]).cuda()
    beta = torch.from_numpy(inp["beta"]).cuda()
    g = torch.Generator(device="cpu").manual_seed(560)
    wg = (torch.rand((B, N, H), generator=g) * 0.5 + 0.5).cuda()
    dg = (torch.rand((B, N, H), generator=g) * 0.1 + 0.9).cuda()
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_BF16)
    ws = torch.empty(max(ia.ia_prefill_gated_workspace_bytes(desc), 16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda")

    def step():
        ia.ia_prefill_fwd_gated(desc, q, k, v, wg, dg, lam, beta, None, o, ws)
    t_start = time.perf_counter()   # half a second of warm-up, as for the prefill step
    while time.perf_counter() - t_start < 0.5:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops, byts = alg_counts(B, N, H, F, D, M)
    byts += 8.0 * B * N * H
    return {"ms_per_step": ms, "tokens_per_s": B * N / (ms * 1e-3),
            "vs_ungated": None if plain_ms is None else ms / plain_ms,
            "mfma_frac": flops / (ms * 1e-3) / BF16_PEAK,
            "hbm_frac": byts / (ms * 1e-3) / HBM_PEAK,
            "scope": "ia_prefill_fwd_gated on the prefill workload (bf16 q, k, v and output; "
                     "chunked MFMA path), whole step"}


def bwd_alg_flops(B, N, H, F, D, M):
    """Algorithmic FLOPs of the backward pass (fp32 VALU): per token, head and mode, the state
    recompute 14 (F + D) and the reverse sweep 44 F + 41 D (a complex multiply counted 6, a
    complex-by-real multiply-add 4)."""
    return float(14 * (F + D) + 44 * F + 41 * D) * M * B * N * H


def bwd_chunked_mfma_flops(B, N, H, F, D, M):
    """FLOPs the chunked backward issues on fp32 MFMA (16x16x4, 2048 FLOP each): per 16-token
    chunk and 16-mode group, the forward sweep's 1.25 (F + D) + 16 instructions and the reverse
    sweep's 1.75 (F + D) + 0.75 (2F + D) + 48 (its products, read off the kernels)."""
    per = 1.25 * (F + D) + 16 + 1.75 * (F + D) + 0.75 * (2 * F + D) + 48
    return per * 2048.0 * ((N + 15) // 16) * (M // 16) * B * H


def bench_backward(torch, ia, inp, bidir=False, steps=5, warmup=2):
    """ia_prefill_bwd over the prefill workload (bf16 q, k, v; fp32 dO), from a zero state
    (both directions for the bidirectional workload): the library's choice of kernels (the
    chunked fp32 MFMA ones on these shapes) and, beside it, the token-sequential kernels."""
    sh = inp["shape"]
    B, H, N, F, D, M = sh["B"], sh["H"], sh["N"], sh["F"], sh["D"], sh["M"]
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).cuda() for n in "qkv")
    lam = torch.from_numpy(inp["lam"]).cuda()
    beta = torch.from_numpy(inp["beta"]).cuda()
    g = torch.Generator(device="cpu").manual_seed(550)
    dO = torch.randn((B, N, H, D), generator=g, dtype=torch.float32).cuda()
    if N > 16384:   # the long genomic sequence: one timed step (a step takes seconds' share)
        steps, warmup = 1, 1
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dl = torch.empty((H, M), dtype=torch.complex64, device="cuda")
    db = torch.empty_like(dl)

    def timed(path):
        desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_F32, bidir=bidir, bwd_path=path)
        ws = torch.empty(ia.ia_prefill_bwd_workspace_bytes(desc), dtype=torch.uint8,
                         device="cuda")

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
        n = ws.numel()
        del ws
        return e0.elapsed_time(e1) / steps * 1e3, n

    chunked = F == D and F in (32, 64, 128) and M % 16 == 0
    us, wsb = timed("auto")
    seq_us, _ = timed("sequential") if chunked else (us, wsb)
    dirs = 2 if bidir else 1
    r = {"us_per_step": us, "tokens_per_s": B * N / (us * 1e-6), "steps": steps,
         "kernels": "chunked fp32 MFMA" if chunked else "token-sequential fp32",
         "dtype": "bf16 in, fp32 state and arithmetic", "workspace_bytes": wsb,
         "sequential_us_per_step": seq_us}
    if chunked:
        fl = bwd_chunked_mfma_flops(B, N, H, F, D, M) * dirs
        r["mfma"] = {"bound": "mfma", "achieved": fl / (us * 1e-6) / 1e12,
                     "peak": FP32_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": fl / (us * 1e-6) / FP32_PEAK, "mfma_flops": fl,
                     "dtype": "f32 (v_mfma_f32_16x16x4_f32)"}
    fl = bwd_alg_flops(B, N, H, F, D, M) * dirs
    r["sequential_alu"] = {"bound": "alu", "achieved": fl / (seq_us * 1e-6) / 1e12,
                           "peak": FP32_PEAK / 1e12, "unit": "TFLOP/s",
                           "frac": fl / (seq_us * 1e-6) / FP32_PEAK, "alg_flops": fl}
    return r


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
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as run in "
                         "half a second, at least 3; the JSON line reports the count)")
    ap.add_argument("--workload", default="1.3b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode measurements (for profiling them); prints their "
                         "JSON object alone")
    ap.add_argument("--block-only", action="store_true",
                    help="run only the block-edge measurements on the 1.3B-shaped tensors (for "
                         "profiling them); prints their JSON object alone")
    ap.add_argument("--gated-only", action="store_true",
                    help="run only the gated prefill measurement on the 1.3B-shaped workload "
                         "(for profiling it); prints its JSON object alone")
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
    if args.decode_only:
        print(json.dumps({"decode": bench_decode(torch, ia, W)}), flush=True)
        return
    if args.block_only:
        inp = WORKLOADS["1.3b"][1](W)
        print(json.dumps({"block_edges": bench_block(torch, ia, W, inp)}), flush=True)
        return
    if args.gated_only:
        inp = WORKLOADS["1.3b"][1](W)
        print(json.dumps({"gated": bench_gated(torch, ia, inp)}), flush=True)
        return
    pf = bench_prefill(args, torch, ia, W)
    dec = None if args.no_decode else bench_decode(torch, ia, W)
    bwd = None
    if not args.no_backward:
        bwd = bench_backward(torch, ia, pf["inp"], bidir=pf["cfg"]["bidirectional"])
    block = gated = None
    if not args.no_decode and args.workload == "1.3b":
        block = bench_block(torch, ia, W, pf["inp"])
        gated = bench_gated(torch, ia, pf["inp"], pf["ms"])
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
        "whole_step": pf["whole"],
        "kernels_ms": pf["kernels_ms"],
        "readout_matrix": pf["readout"],
        "decode": dec,
        "block_edges": block,
        "gated": gated,
        "backward": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
