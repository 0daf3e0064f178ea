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


@pytest.mark.parametrize("path", ["chunked", "sequential"])
@pytest.mark.parametrize("bidir", [False, True])
def test_graph_backward(bidir, path):
    """The backward in a graph, replayed: the chunked kernels, and the token-sequential ones
    (few slices: several sequence segments and their carries)."""
    import torch
    ia = _ia()
    B, H, N, F, D, M = 1, 2, 600, 64, 64, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="bf16", seed=720)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    dO = dev(np.random.default_rng(721).standard_normal((B, N, H, D)).astype(np.float32))
    desc = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_F32, bidir=bidir, bwd_path=path)
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

    tag(f"graph backward bidir={bidir} path={path}")
    run()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    _replays(torch, run, reset, outs, eager)


@pytest.mark.parametrize("fused", [False, True])
def test_graph_block_decode_stack(fused):
    """Three blocks decoding four tokens in one graph.  Per token and layer: the prologue
    (convolution state in two buffers taken in turn, RoPE at the token's position, the
    normalisation), ia_decode_step with identity features, the output gate in place -- or, fused,
    ia_block_decode_step doing all three; layer l > 0 takes layer l-1's gated output as its v,
    so the graph's order matters.  Replays equal the eager run exactly; the eager run equals the
    oracle's prologue, brute-force layer and gate, layer by layer on that layer's own inputs."""
    import torch
    import oracle.block as blk
    from oracle import brute
    from helpers import TOL_BF16, host, report, rowrel
    ia = _ia()
    B, H, F, D, M, Wd, L, T, pos0 = 2, 4, 64, 64, 16, 4, 3, 4, 7
    tb = torch.bfloat16
    r = np.random.default_rng(730)
    bf = lambda *shape, s=1.0: W.round_bf16((r.standard_normal(shape) * s).astype(np.float32))
    qs = [bf(T, B, 1, H, F, s=0.5) for _ in range(L)]
    ks = [bf(T, B, 1, H, F, s=0.5) for _ in range(L)]
    v0 = bf(T, B, 1, H, D)
    gs = [bf(T, B, 1, H, D) for _ in range(L)]
    convs = [tuple((r.standard_normal((H, C, Wd)) * 0.4).astype(np.float32) for C in (F, F, D))
             for _ in range(L)]
    norms = [((1 + 0.1 * r.standard_normal((H, F + D))).astype(np.float32),
              (0.05 * r.standard_normal((H, F + D))).astype(np.float32)) for _ in range(L)]
    lams = [W.s4d_lin(np.exp(r.uniform(np.log(1e-3), np.log(1e-1), H)), M) for _ in range(L)]
    beta = np.ones((H, M), np.complex64)

    qd = [[dev(x[t], tb) for t in range(T)] for x in qs]
    kd = [[dev(x[t], tb) for t in range(T)] for x in ks]
    gd = [[dev(x[t], tb) for t in range(T)] for x in gs]
    v0d = [dev(v0[t], tb) for t in range(T)]
    convd = [tuple(dev(w) for w in c) for c in convs]    # kept alive: params hold addresses
    normd = [tuple(dev(w) for w in n) for n in norms]
    ps = [[ia.block_params(convd[l], 1e4, pos0 + t, normd[l]) for t in range(T)]
          for l in range(L)]
    lamd, betad = [dev(x) for x in lams], dev(beta)
    d1 = ia.make_desc(B, H, 1, F, D, M, ia.IA_BF16, ia.IA_BF16)
    dd = ia.make_desc(B, H, 1, F, D, M, ia.IA_BF16, ia.IA_BF16, identity_features=True)
    sts = [ia.new_state(B, H, M, F, D) for _ in range(L)]
    cs = [[torch.zeros((B, H, Wd - 1, 2 * F + D), device="cuda") for _ in range(2)]
          for _ in range(L)]
    feats = [tuple(torch.empty((B, 1, H, C), dtype=tb, device="cuda") for C in (F, F, D))
             for _ in range(L)]
    out = [torch.empty((T, B, 1, H, D), dtype=tb, device="cuda") for _ in range(L)]

    def run():
        for t in range(T):
            for l in range(L):
                vin = v0d[t] if l == 0 else out[l - 1][t]
                if fused:
                    ia.ia_block_decode_step(d1, ps[l][t], qd[l][t][:, 0], kd[l][t][:, 0],
                                            vin[:, 0], cs[l][t % 2], cs[l][1 - t % 2],
                                            gd[l][t][:, 0], lamd[l], betad, sts[l],
                                            out[l][t][:, 0])
                    continue
                fq, fk, vo = feats[l]
                ia.ia_block_prologue(d1, ps[l][t], qd[l][t], kd[l][t], vin, cs[l][t % 2],
                                     cs[l][1 - t % 2], fq, fk, vo)
                ia.ia_decode_step(dd, fq[:, 0], fk[:, 0], vo[:, 0], lamd[l], betad, sts[l],
                                  out[l][t][:, 0])
                ia.ia_block_gate(d1, out[l][t], gd[l][t], out[l][t])

    def reset():
        for l in range(L):
            for x in sts[l] + tuple(cs[l]):
                x.zero_()

    tag(f"graph block decode stack fused={fused}")
    reset()
    run()
    torch.cuda.synchronize()
    outputs = out + [x for l in range(L) for x in sts[l] + tuple(cs[l])]
    eager = [x.clone() for x in outputs]

    # the oracle, layer by layer on the layer's inputs as the GPU saw them
    seq = lambda a: np.transpose(a[:, :, 0], (1, 0, 2, 3)).astype(np.float64)   # [B,T,H,C]
    for l in range(L):
        vin = v0 if l == 0 else host(out[l - 1])
        fq, fk, vo, _ = blk.prologue(seq(qs[l]), seq(ks[l]), seq(vin), convs[l], None, 1e4,
                                     pos0, norms[l], 1e-6)
        o = np.empty((B, T, H, D))
        for b in range(B):
            for h in range(H):
                o[b, :, h] = brute.layer(fq[b, :, h], fk[b, :, h], vo[b, :, h], lams[l][h],
                                         beta[h], features_given=True)[0]
        err = rowrel(seq(host(out[l])), blk.gate(o, seq(gs[l])))
        report(f"graph block decode stack fused={fused}, layer {l}", err)
        assert err < TOL_BF16, (l, err)

    for x in out:
        x.zero_()
    _replays(torch, run, reset, outputs, eager)
