"""GPU parity of the block's edges (ia_block_prologue, ia_block_gate) against oracle/block.py,
and of the whole block (prologue, the layer with identity features on the chunked path, the
output gate) against the oracle's composition with the brute-force layer.  Tolerances:
row-wise relative 1e-4 with fp32 data, 1e-2 for bf16 outputs (one bf16 rounding, 2^-9, of
each output element); 2e-2 for the whole block with bf16 inputs (the layer's bound)."""
import numpy as np
import pytest

import ia_workloads as W
import oracle.block as blk
from oracle import brute
from helpers import TOL_BF16, dev, host, report, rowrel, tag

pytestmark = pytest.mark.gpu


def _ia():
    import ssm_sequence_mixer_amd as ia
    return ia


def _params(H, F, D, Wd, seed, rope=True, norm=True):
    r = np.random.default_rng(seed)
    conv = None
    if Wd > 0:
        conv = tuple((r.standard_normal((H, C, Wd)) * (0.8 / np.sqrt(Wd))).astype(np.float32)
                     for C in (F, F, D))
    nrm = None
    if norm:
        nrm = ((1.0 + 0.1 * r.standard_normal((H, F + D))).astype(np.float32),
               (0.05 * r.standard_normal((H, F + D))).astype(np.float32))
    return conv, (1e4 if rope else 0.0), nrm


def _raw(B, N, H, F, D, dtype, seed, std=1.0):
    r = np.random.default_rng(seed)
    x = [r.standard_normal((B, N, H, C)).astype(np.float32) * std for C in (F, F, D)]
    if dtype == "bf16":
        x = [W.round_bf16(a) for a in x]
    return x


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _run(ia, q, k, v, conv, rope, nrm, dtype, state=None, pos0=0):
    import torch
    t = _tdt(dtype)
    c = None if conv is None else tuple(dev(w) for w in conv)
    n = None if nrm is None else tuple(dev(w) for w in nrm)
    st = None if state is None else dev(state)
    out = ia.block_prologue(dev(q, t), dev(k, t), dev(v, t), conv=c, state=st, rope_base=rope,
                            pos0=pos0, norm=n)
    torch.cuda.synchronize()
    return tuple(None if x is None else host(x) for x in out)


@pytest.mark.parametrize("shape", [(1, 2, 100, 32, 32, 4), (2, 3, 130, 64, 32, 3),
                                   (1, 2, 200, 128, 128, 4), (1, 2, 70, 32, 64, 1),
                                   (1, 1, 1, 32, 32, 8), (2, 2, 65, 64, 64, 0),
                                   (1, 2, 150, 32, 32, 2), (1, 1, 90, 64, 32, 5),
                                   (1, 1, 40, 32, 256, 6), (1, 1, 20, 256, 32, 7)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("opts", ["all", "no_rope", "no_norm"])
def test_prologue_matches_oracle(shape, dtype, opts):
    """Every stage on: convolution (W taps; 0 = none), RoPE from position 5, the
    normalisation; then without RoPE, without the normalisation.  Ragged token counts over
    the 64-token blocks, every output element and the new convolution state."""
    ia = _ia()
    B, H, N, F, D, Wd = shape
    q, k, v = _raw(B, N, H, F, D, dtype, 300 + N + F)
    conv, rope, nrm = _params(H, F, D, Wd, 301, rope=opts != "no_rope", norm=opts != "no_norm")
    tag(f"block prologue {shape} {dtype} {opts}")
    fq, fk, vo, st = _run(ia, q, k, v, conv, rope, nrm, dtype, pos0=5)
    rq, rk, rv, rst = blk.prologue(q, k, v, conv, None, rope, 5, nrm, 1e-6)
    tol = 1e-2 if dtype == "bf16" else 1e-4
    errs = [rowrel(fq, rq), rowrel(fk, rk), rowrel(vo, rv)]
    report(f"block prologue {shape} {dtype} {opts}", max(errs))
    assert max(errs) < tol, errs
    if Wd > 1:
        np.testing.assert_allclose(st, rst, rtol=1e-6, atol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prologue_far_positions(dtype):
    """RoPE at positions up to the largest one the entry point takes (2^31 - 1): each
    token's angle reduced from its own position."""
    ia = _ia()
    B, H, N, F, D, Wd = 1, 2, 140, 64, 32, 3
    q, k, v = _raw(B, N, H, F, D, dtype, 310)
    conv, rope, nrm = _params(H, F, D, Wd, 311)
    for pos0 in (1_000_003, 2**31 - N):
        tag(f"block prologue far positions {dtype} pos0={pos0}")
        fq, fk, vo, _ = _run(ia, q, k, v, conv, rope, nrm, dtype, pos0=pos0)
        rq, rk, rv, _ = blk.prologue(q, k, v, conv, None, rope, pos0, nrm, 1e-6)
        errs = [rowrel(fq, rq), rowrel(fk, rk), rowrel(vo, rv)]
        report(f"block prologue far positions {dtype} pos0={pos0}", max(errs))
        assert max(errs) < (1e-2 if dtype == "bf16" else 1e-4), errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prologue_state_carry_and_decode_steps(dtype):
    """Two calls carrying the convolution state and the position equal one call exactly;
    then four single-token calls (the decode form) continue it exactly."""
    ia = _ia()
    B, H, N, F, D, Wd = 2, 2, 150, 64, 64, 4
    q, k, v = _raw(B, N + 4, H, F, D, dtype, 320)
    conv, rope, nrm = _params(H, F, D, Wd, 321)
    tag(f"block prologue carry {dtype}")
    whole = _run(ia, q, k, v, conv, rope, nrm, dtype)
    a = _run(ia, q[:, :70], k[:, :70], v[:, :70], conv, rope, nrm, dtype)
    b = _run(ia, q[:, 70:N + 4], k[:, 70:N + 4], v[:, 70:N + 4], conv, rope, nrm, dtype,
             state=a[3], pos0=70)
    for i in range(3):
        np.testing.assert_array_equal(np.concatenate([a[i], b[i]], axis=1), whole[i])
    np.testing.assert_array_equal(b[3], whole[3])
    head = _run(ia, q[:, :N], k[:, :N], v[:, :N], conv, rope, nrm, dtype)
    st = head[3]
    for t in range(N, N + 4):
        step = _run(ia, q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], conv, rope, nrm, dtype,
                    state=st, pos0=t)
        for i in range(3):
            np.testing.assert_array_equal(step[i][:, 0], whole[i][:, t])
        st = step[3]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_gate_matches_oracle(dtype):
    import torch
    ia = _ia()
    r = np.random.default_rng(330)
    o = r.standard_normal((2, 37, 3, 64)).astype(np.float32)
    g = (r.standard_normal((2, 37, 3, 64)) * 3).astype(np.float32)
    if dtype == "bf16":
        o, g = W.round_bf16(o), W.round_bf16(g)
    t = _tdt(dtype)
    tag(f"block gate {dtype}")
    od, gd = dev(o, t), dev(g, t)
    out = host(ia.block_gate(od, gd))
    ref = blk.gate(o, g)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    assert rowrel(out, ref) < tol
    ia.block_gate(od, gd, out=od)   # in place
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(od), out)


def test_whole_block_matches_oracle():
    """Prologue, the chunked layer with identity features (bf16, chunk 64, several segments),
    then the output gate, against oracle.block's prologue and gate around the brute-force
    layer with the features given."""
    import torch
    ia = _ia()
    B, H, N, F, D, M, Wd = 1, 4, 96, 64, 64, 16, 4
    q, k, v = _raw(B, N, H, F, D, "bf16", 340, std=0.5)
    g = W.round_bf16(np.random.default_rng(341).standard_normal((B, N, H, D)).astype(np.float32))
    conv, rope, nrm = _params(H, F, D, Wd, 342)
    lam = W.s4d_lin(np.exp(np.random.default_rng(343).uniform(np.log(1e-3), np.log(1e-1), H)), M)
    beta = np.ones((H, M), np.complex64)
    tb = torch.bfloat16
    tag("whole block: prologue, layer with identity features, gate")
    fq, fk, vo, _ = ia.block_prologue(dev(q, tb), dev(k, tb), dev(v, tb),
                                      conv=tuple(dev(w) for w in conv), rope_base=rope,
                                      norm=tuple(dev(w) for w in nrm), M=M)
    # the entry point itself with neither convolution state (NULL in, NULL out)
    conv_d, nrm_d = tuple(dev(w) for w in conv), tuple(dev(w) for w in nrm)   # kept alive
    p = ia.block_params(conv_d, rope, 0, nrm_d)
    d = ia.make_desc(B, H, N, F, D, M, ia.IA_BF16, ia.IA_BF16)
    alt = tuple(torch.empty_like(x) for x in (fq, fk, vo))
    ia.ia_block_prologue(d, p, dev(q, tb), dev(k, tb), dev(v, tb), None, None, *alt)
    torch.cuda.synchronize()
    for x, y in zip(alt, (fq, fk, vo)):
        assert torch.equal(x, y)
    o = ia.prefill(fq, fk, vo, dev(lam), dev(beta), out_dtype=tb, identity_features=True)
    out = host(ia.block_gate(o, dev(g, tb)))
    torch.cuda.synchronize()
    # the oracle's chain, on the GPU prologue's bf16 outputs for the layer (the layer's bound
    # covers its own rounding; the prologue is compared separately above) ...
    lf = [host(x) for x in (fq, fk, vo)]
    ref = np.empty((B, N, H, D))
    for b in range(B):
        for h in range(H):
            ref[b, :, h] = brute.layer(lf[0][b, :, h], lf[1][b, :, h], lf[2][b, :, h], lam[h],
                                       beta[h], features_given=True)[0]
    err = rowrel(out, blk.gate(ref, g))
    report("whole block, layer and gate", err)
    assert err < TOL_BF16
    # ... and the oracle's own prologue against the GPU's, so the chain is covered end to end
    rq, rk, rv, _ = blk.prologue(q, k, v, conv, None, rope, 0, nrm, 1e-6)
    assert max(rowrel(lf[0], rq), rowrel(lf[1], rk), rowrel(lf[2], rv)) < 1e-2


def _step_inputs(B, H, T, F, D, M, Wd, dtype, seed):
    r = np.random.default_rng(seed)
    raw = [(r.standard_normal((T, B, H, C)) * 0.7).astype(np.float32) for C in (F, F, D)]
    g = r.standard_normal((T, B, H, D)).astype(np.float32)
    if dtype == "bf16":
        raw, g = [W.round_bf16(a) for a in raw], W.round_bf16(g)
    lam = W.s4d_lin(np.exp(r.uniform(np.log(1e-3), np.log(1e-1), H)), M)
    return raw, g, lam


def _step_oracle(raw, g, lam, conv, rope, pos0, nrm, gated, no_den=False):
    """The oracle's prologue over the T tokens, the brute-force layer from zero state with the
    features given, the gate: [T, B, H, D]."""
    T, B, H, F = raw[0].shape
    D = raw[2].shape[3]
    seq = [np.transpose(a, (1, 0, 2, 3)).astype(np.float64) for a in raw]   # [B,T,H,C]
    fq, fk, vo, _ = blk.prologue(*seq, conv, None, rope, pos0, nrm, 1e-6)
    o = np.empty((B, T, H, D))
    beta = np.ones(lam.shape[1], np.complex128)
    for b in range(B):
        for h in range(H):
            res = brute.layer(fq[b, :, h], fk[b, :, h], vo[b, :, h], lam[h], beta,
                              features_given=True)
            o[b, :, h] = res[1] if no_den else res[0]
    if gated:
        o = blk.gate(o, np.transpose(g, (1, 0, 2, 3)))
    return np.transpose(o, (1, 0, 2, 3))


def _run_steps(ia, raw, g, lam, conv, rope, pos0, nrm, dtype, gated, fused, no_den=False):
    """T decode tokens through ia_block_decode_step (fused) or through ia_block_prologue,
    ia_decode_step with identity features and ia_block_gate; returns the outputs [T,B,H,D]
    (float) and the final convolution state."""
    import torch
    t_dt = _tdt(dtype)
    T, B, H, F = raw[0].shape
    D, M = raw[2].shape[3], lam.shape[1]
    Wd = 0 if conv is None else conv[0].shape[2]
    c = None if conv is None else tuple(dev(w) for w in conv)
    n = None if nrm is None else tuple(dev(w) for w in nrm)
    lamd, betad = dev(lam), dev(np.ones((H, M), np.complex64))
    st = ia.new_state(B, H, M, F, D)
    cs = [torch.zeros((B, H, max(Wd - 1, 1), 2 * F + D), device="cuda") for _ in range(2)]
    d1 = ia.make_desc(B, H, 1, F, D, M, ia.dtype_code(t_dt), ia.dtype_code(t_dt), no_den=no_den)
    di = ia.make_desc(B, H, 1, F, D, M, ia.dtype_code(t_dt), ia.dtype_code(t_dt), no_den=no_den,
                      identity_features=True)
    outs = []
    for t in range(T):
        p = ia.block_params(c, rope, pos0 + t, n)
        sin, sout = (cs[t % 2], cs[1 - t % 2]) if Wd > 1 else (None, None)
        q, k, v = (dev(a[t], t_dt) for a in raw)
        gt = dev(g[t], t_dt) if gated else None
        out = torch.empty((B, H, D), dtype=t_dt, device="cuda")
        if fused:
            ia.ia_block_decode_step(d1, p, q, k, v, sin, sout, gt, lamd, betad, st, out)
        else:
            f = tuple(torch.empty_like(x) for x in (q, k, v))
            ia.ia_block_prologue(d1, p, q, k, v, sin, sout, *f)
            ia.ia_decode_step(di, *f, lamd, betad, st, out)
            if gated:
                ia.ia_block_gate(d1, out, gt, out)
        torch.cuda.synchronize()
        outs.append(host(out))
    return np.stack(outs), (host(cs[T % 2]) if Wd > 1 else None)


# (B, H, F, D, M, W): row-parallel decode kernel (M <= 64 and M = 80), the mode-looping one
# (F = 256, and 2048 slices), the latter with two channel pairs per thread at F = Dv = 256
STEP_SHAPES = [(2, 3, 64, 64, 16, 4), (1, 2, 128, 128, 64, 3), (1, 1, 32, 128, 80, 2),
               (1, 2, 256, 64, 16, 4), (1, 1, 256, 256, 32, 8), (128, 16, 32, 32, 16, 4)]


@pytest.mark.parametrize("shape", STEP_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_decode_step_matches_oracle(shape, dtype):
    """Five tokens through the fused block step from zero states (RoPE from position 11, the
    normalisation, the gate) against the oracle's prologue, layer and gate, and against the
    three-call route; the final convolution state equal to the three-call route's."""
    ia = _ia()
    B, H, F, D, M, Wd = shape
    T = 3 if B * H > 1000 else 5
    raw, g, lam = _step_inputs(B, H, T, F, D, M, Wd, dtype, 400 + F + D + M)
    conv, rope, nrm = _params(H, F, D, Wd, 401)
    tag(f"block decode step {shape} {dtype}")
    got, st = _run_steps(ia, raw, g, lam, conv, rope, 11, nrm, dtype, True, True)
    three, st3 = _run_steps(ia, raw, g, lam, conv, rope, 11, nrm, dtype, True, False)
    ref = _step_oracle(raw, g, lam, conv, rope, 11, nrm, True)
    tol = TOL_BF16 if dtype == "bf16" else 2e-3
    err, err3 = rowrel(got, ref), rowrel(got, three)
    report(f"block decode step {shape} {dtype}", err)
    assert err < tol, (err, err3)
    assert err3 < tol, (err, err3)
    if st is not None:
        np.testing.assert_array_equal(st, st3)


@pytest.mark.parametrize("opts", ["no_gate", "no_rope_no_norm", "no_conv", "one_tap", "no_den"])
def test_block_decode_step_options(opts):
    ia = _ia()
    B, H, F, D, M = 2, 2, 64, 32, 16
    Wd = {"no_conv": 0, "one_tap": 1}.get(opts, 3)
    raw, g, lam = _step_inputs(B, H, 4, F, D, M, Wd, "f32", 410)
    conv, rope, nrm = _params(H, F, D, Wd, 411, rope=opts != "no_rope_no_norm",
                              norm=opts != "no_rope_no_norm")
    gated, no_den = opts != "no_gate", opts == "no_den"
    tag(f"block decode step {opts}")
    got, _ = _run_steps(ia, raw, g, lam, conv, rope, 0, nrm, "f32", gated, True, no_den)
    ref = _step_oracle(raw, g, lam, conv, rope, 0, nrm, gated, no_den)
    err = rowrel(got, ref)
    report(f"block decode step {opts}", err)
    assert err < 2e-3, err
