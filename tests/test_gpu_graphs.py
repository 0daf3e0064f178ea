"""Graph capture of the C ABI calls (hipGraphs through torch.cuda.CUDAGraph): decode steps,
the chunked prefill (several segments: state-only pass with the tables, carry, output pass)
and the backward.  Each graph is captured once after an eager warm-up, then replayed three
times with eager work (state resets, unrelated kernels, synchronizations) between replays;
every replay must equal the eager result exactly, since every kernel sums in a fixed order.
"""
import numpy as np
import pytest

import ia_workloads as W
from helpers import dev, tag

pytestmark = pytest.mark.gpu


def _ia():
    import ssm_sequence_mixer_amd as ia
    return ia


def _replays(torch, fn, reset, outputs, eager):
    """Capture fn, then replay 3 times; after each replay compare `outputs` with `eager`."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        reset()
        torch.randn(1 << 16, device="cuda").sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(range(len(outputs)), outputs, eager):
            assert torch.equal(got, want), f"replay {r}: output {name} differs from eager"
    del g


@pytest.mark.parametrize("B", [2, 512])
def test_graph_decode_steps(B):
    """Row-parallel kernel (B=2, H=4: 8 slices) and mode-looping kernel (B=512: 2048 slices,
    eight per compute unit); 6 steps per graph."""
    import torch
    ia = _ia()
    H, F, D, M, steps = 4, 128, 128, 64, 6
    inp = W.make_inputs(B, H, steps, F, D, M, dtype="bf16", seed=700 + B)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    desc = ia.make_desc(B, H, 1, F, D, M, ia.IA_BF16, ia.IA_F32)
    st0 = ia.new_state(B, H, M, F, D)
    pre = W.make_inputs(B, H, 16, F, D, M, dtype="bf16", seed=701)
    ia.prefill(dev(pre["q"], torch.bfloat16), dev(pre["k"], torch.bfloat16),
               dev(pre["v"], torch.bfloat16), lam, beta, state=st0, want_output=False)
    st = tuple(x.clone() for x in st0)
    o = torch.empty((steps, B, H, D), dtype=torch.float32, device="cuda")
    qt = [q[:, t].contiguous() for t in range(steps)]
    kt = [k[:, t].contiguous() for t in range(steps)]
    vt = [v[:, t].contiguous() for t in range(steps)]

    def run():
        for t in range(steps):
            ia.ia_decode_step(desc, qt[t], kt[t], vt[t], lam, beta, st, o[t])

    def reset():
        for a, b in zip(st, st0):
            a.copy_(b)

    tag(f"graph decode B={B}")
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone()] + [x.clone() for x in st]
    o.zero_()
    _replays(torch, run, reset, [o] + list(st), eager)


def test_graph_chunked_prefill_with_segments():
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 4, 1500, 128, 128, 64
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=710)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_BF16)
    ws = torch.empty(max(ia.ia_prefill_workspace_bytes(desc), 16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda")
    st0 = ia.new_state(B, H, M, F, D)
    st = tuple(x.clone() for x in st0)

    def run():
        ia.ia_prefill_fwd(desc, q, k, v, lam, beta, st, o, ws)

    def reset():
        for a, b in zip(st, st0):
            a.copy_(b)

    tag("graph chunked prefill")
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone()] + [x.clone() for x in st]
    o.zero_()
    _replays(torch, run, reset, [o] + list(st), eager)


@pytest.mark.parametrize("bidir", [False, True])
def test_graph_backward(bidir):
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 2, 600, 64, 64, 32   # few slices: several sequence segments
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=720)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    dO = dev(np.random.default_rng(721).standard_normal((B, N, H, D)).astype(np.float32))
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_F32, bidir=bidir)
    ws = torch.empty(ia.ia_prefill_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dl = torch.empty((H, M), dtype=torch.complex64, device="cuda")
    db = torch.empty_like(dl)
    outs = [dq, dk, dv, dl, db]

    def run():
        ia.ia_prefill_bwd(desc, q, k, v, lam, beta, None, dO, dq, dk, dv, dl, db, None, ws)

    def reset():
        for x in outs:
            x.zero_()

    tag(f"graph backward bidir={bidir}")
    run()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    _replays(torch, run, reset, outs, eager)
