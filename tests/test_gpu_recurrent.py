"""GPU parity of the token-by-token kernels (decode step, fp32 prefill) against the oracle.

All inputs are seeded (ia_workloads); the oracle receives the very values the GPU receives.
"""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from helpers import TOL_BF16, TOL_F32, dev, host, report, rowrel, state_rel, tag

pytestmark = pytest.mark.gpu


def _lib():
    import ssm_sequence_mixer_amd as ia
    return ia


def _torch():
    import torch
    return torch


def _oracle_state(B, H, F, D, M, lam, beta, seed):
    """A non-trivial state: the oracle's state after 9 random tokens."""
    inp = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=seed, std=0.5)
    _, _, _, st = oracle.prefill(inp["q"], inp["k"], inp["v"], lam, beta)
    return st


@pytest.mark.parametrize("in_dtype,out_dtype", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_decode_steps_match_oracle(in_dtype, out_dtype):
    torch = _torch()
    ia = _lib()
    B, H, F, D, M, steps = 2, 3, 32, 48, 16, 5
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=in_dtype, seed=11)
    lam, beta = inp["lam"], inp["beta"] * np.complex64(0.7 - 0.2j)
    st_ref = _oracle_state(B, H, F, D, M, lam, beta, seed=12)
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)  # both sides continue from the complex64 state
    for t in range(steps):
        tag(f"decode step {t} {in_dtype}->{out_dtype}")
        o = ia.decode(dev(inp["q"][:, t], tdt[in_dtype]), dev(inp["k"][:, t], tdt[in_dtype]),
                      dev(inp["v"][:, t], tdt[in_dtype]), dev(lam), dev(beta), st,
                      out_dtype=tdt[out_dtype])
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        tol = TOL_F32 if out_dtype == "f32" else TOL_BF16
        assert rowrel(host(o), o_ref) < tol
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("shape", [(32, 32, 16), (32, 128, 64), (64, 64, 128), (128, 32, 16),
                                   (64, 128, 32), (128, 128, 64), (128, 128, 128)])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_decode_row_kernel_shapes(shape, in_dtype):
    """Decode at the row widths the row-parallel kernel takes (F, Dv in {32, 64, 128}),
    including passes that cover more rows than there are modes (F=32, M=16)."""
    torch = _torch()
    ia = _lib()
    F, D, M = shape
    B, H, steps = 3, 2, 3
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=in_dtype, seed=F + D + M)
    lam, beta = inp["lam"], inp["beta"]
    st_ref = _oracle_state(B, H, F, D, M, lam, beta, seed=M + 1)
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    for t in range(steps):
        tag(f"decode rows F={F} D={D} M={M} {in_dtype} step {t}")
        o = ia.decode(dev(inp["q"][:, t], tdt[in_dtype]), dev(inp["k"][:, t], tdt[in_dtype]),
                      dev(inp["v"][:, t], tdt[in_dtype]), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        assert rowrel(host(o), o_ref) < TOL_F32
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("BH", [(1, 16), (3, 8), (4, 16), (8, 16), (1, 5)])
@pytest.mark.parametrize("M", [16, 32, 64])
@pytest.mark.parametrize("FD", [(128, 128), (64, 32), (32, 64)])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_decode_rows_few_slices(BH, M, FD, in_dtype):
    """The row-parallel kernel at few slices (5 to 128) and the row widths whose lane sums take
    one, two or four 16-lane rows (F/2 = 64, 32, 16 lanes per state row): outputs and every
    state tensor against the oracle over three steps from a non-zero state."""
    torch = _torch()
    ia = _lib()
    B, H = BH
    F, D = FD
    steps = 3
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=in_dtype, seed=900 + B * H + M + F)
    lam, beta = inp["lam"], inp["beta"] * np.complex64(0.9 + 0.3j)
    st_ref = _oracle_state(B, H, F, D, M, lam, beta, seed=901 + M)
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    for t in range(steps):
        tag(f"decode rows B={B} H={H} F={F} D={D} M={M} {in_dtype} step {t}")
        o = ia.decode(dev(inp["q"][:, t], tdt[in_dtype]), dev(inp["k"][:, t], tdt[in_dtype]),
                      dev(inp["v"][:, t], tdt[in_dtype]), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        assert rowrel(host(o), o_ref) < TOL_F32
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_decode_mode_looping_kernel_many_slices(in_dtype):
    """2048 slices (B=128, H=16) at F = Dv = 128, M = 16: eight slices per compute unit take
    the mode-looping kernel.  Outputs and state over two steps from a non-zero state."""
    torch = _torch()
    ia = _lib()
    B, H, F, D, M, steps = 128, 16, 128, 128, 16, 2
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    inp = W.make_inputs(B, H, steps, F, D, M, dtype=in_dtype, seed=950)
    lam, beta = inp["lam"], inp["beta"]
    st_ref = _oracle_state(B, H, F, D, M, lam, beta, seed=951)
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    for t in range(steps):
        tag(f"decode mode-looping B={B} H={H} {in_dtype} step {t}")
        o = ia.decode(dev(inp["q"][:, t], tdt[in_dtype]), dev(inp["k"][:, t], tdt[in_dtype]),
                      dev(inp["v"][:, t], tdt[in_dtype]), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        assert rowrel(host(o), o_ref) < TOL_F32
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


def test_fp32_prefill_tiny_workload():
    """The tiny fp32 workload: B=H=1, N=256, F=Dv=M=16, dt=0.01, beta=1; outputs and state."""
    torch = _torch()
    ia = _lib()
    inp = W.tiny()
    tag("fp32 prefill tiny")
    st = ia.new_state(1, 1, 16, 16, 16)
    o = ia.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]),
                   dev(inp["beta"]), state=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, _, den_ref, st_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"],
                                               inp["beta"])
    assert np.all(den_ref > 10 * 1e-6)
    assert rowrel(host(o), o_ref) < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("N", [1, 63, 130])
def test_fp32_prefill_ragged_and_resume(N):
    torch = _torch()
    ia = _lib()
    B, H, F, D, M = 2, 2, 32, 16, 32
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=20 + N)
    q, k, v = (dev(inp[n]) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    tag(f"fp32 prefill N={N}")
    st = ia.new_state(B, H, M, F, D)
    o = ia.prefill(q, k, v, lam, beta, state=st, out_dtype=torch.float32)
    o_ref, _, _, st_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
    torch.cuda.synchronize()
    assert rowrel(host(o), o_ref) < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32
    # state-only prefill of a prefix, then the rest from that state, equals the whole
    if N > 1:
        s = N // 2
        st2 = ia.new_state(B, H, M, F, D)
        ia.prefill(q[:, :s].contiguous(), k[:, :s].contiguous(), v[:, :s].contiguous(), lam,
                   beta, state=st2, want_output=False)
        o2 = ia.prefill(q[:, s:].contiguous(), k[:, s:].contiguous(), v[:, s:].contiguous(),
                        lam, beta, state=st2, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert rowrel(host(o2), o_ref[:, s:]) < TOL_F32
        assert state_rel(tuple(host(x) for x in st2), st_ref) < TOL_F32


def test_fp32_bidirectional():
    torch = _torch()
    ia = _lib()
    B, H, N, F, D, M = 1, 2, 45, 16, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=31)
    tag("fp32 bidir")
    o = ia.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["lam"]),
                   dev(inp["beta"]), bidir=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref = oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
    assert rowrel(host(o), o_ref) < TOL_F32


def test_decode_forced_clamp():
    """beta = i with real lambda drives Re(den) below zero: o_t = num / clamp."""
    torch = _torch()
    ia = _lib()
    B, H, F, D, M = 1, 1, 16, 16, 16
    lam = np.full((H, M), 0.9, np.complex64)
    beta = np.full((H, M), 1j, np.complex64)
    inp = W.make_inputs(B, H, 3, F, D, M, dtype="f32", seed=41)
    st = ia.new_state(B, H, M, F, D)
    st_ref = tuple(np.zeros(s, np.complex128) for s in ((B, H, M, F), (B, H, M, D), (B, H, M)))
    for t in range(3):
        tag(f"decode clamp step {t}")
        o = ia.decode(dev(inp["q"][:, t]), dev(inp["k"][:, t]), dev(inp["v"][:, t]), dev(lam),
                      dev(beta), st)
        o_ref, st_ref = oracle.decode_step(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], lam,
                                           beta, st_ref)
        torch.cuda.synchronize()
        assert np.all(np.abs(o_ref) > 1e3)  # the clamp was hit
        assert rowrel(host(o), o_ref) < TOL_F32


@pytest.mark.parametrize("Bd", [1, 16, 64])
def test_decode_1p3b_workload_all_steps(Bd):
    """The decode workload in full: at the 1.3B-shaped layer (H=16, F=Dv=128, M=64), a
    32-token chunked prefill of a random prefix, then all 256 decode steps, at the benchmark's
    batch sizes (16, 256 and 1024 slices, all on the row-parallel kernel).
    Every step's output of every (b, h) slice, and the state after the prefix and after the
    last step, against the oracle's recurrence over all 288 tokens (the scan the decode steps
    continue)."""
    torch = _torch()
    ia = _lib()
    steps, prefix = 256, 32
    wl = W.decode(Bd, steps=steps, prefix=prefix)
    pre, stp = wl["prefix"], wl["steps"]
    lam, beta = wl["lam"], wl["beta"]
    bf = torch.bfloat16
    tag(f"decode 1.3b B={Bd} prefix")
    st = ia.new_state(Bd, 16, 64, 128, 128)
    ia.prefill(dev(pre["q"], bf), dev(pre["k"], bf), dev(pre["v"], bf), dev(lam), dev(beta),
               state=st, want_output=False)
    torch.cuda.synchronize()
    st_pre = tuple(host(s) for s in st)
    sq, sk, sv = (dev(stp[n], bf) for n in "qkv")
    lam_d, beta_d = dev(lam), dev(beta)
    o = torch.empty((steps, Bd, 16, 128), dtype=torch.float32, device="cuda")
    tag(f"decode 1.3b B={Bd} {steps} steps")
    for t in range(steps):
        ia.decode(sq[t], sk[t], sv[t], lam_d, beta_d, st, o_t=o[t])
    torch.cuda.synchronize()
    o = host(o)
    # the oracle: one recurrence per slice over the prefix and the steps
    seq = {n: np.concatenate([pre[n], np.moveaxis(stp[n], 0, 1)], axis=1) for n in "qkv"}
    _, _, _, st_ref_pre = oracle.prefill(pre["q"], pre["k"], pre["v"], lam, beta, threads=16)
    o_ref, _, _, st_ref = oracle.prefill(seq["q"], seq["k"], seq["v"], lam, beta, threads=16)
    e_pre = state_rel(st_pre, st_ref_pre)
    report(f"decode 1.3b B={Bd} prefix state (chunked bf16 path)", e_pre)
    worst = max(rowrel(o[t], o_ref[:, prefix + t]) for t in range(steps))
    report(f"decode 1.3b B={Bd} all {steps} steps, every slice", worst)
    e_st = state_rel(tuple(host(s) for s in st), st_ref)
    report(f"decode 1.3b B={Bd} state after the last step", e_st)
    assert e_pre < TOL_BF16 and worst < TOL_BF16 and e_st < TOL_BF16


@pytest.mark.parametrize("shape", [(64, 32, 16), (16, 240, 48), (128, 64, 128), (256, 256, 128)])
def test_shapes_outside_the_chunk_kernels(shape):
    """Shapes the chunked kernels do not take (F != Dv, widths 240/256, M=128; 256/256/128 is
    the largest the library accepts): a bf16 prefill is refused (IA_ERR_UNSUPPORTED, no slow
    fallback); the same bf16-exact values in fp32 run the token-sequential prefill, then two
    bf16 decode steps (the mode-looping kernel), outputs and state.  The oracle sees the same
    values, so fp32 arithmetic sets the bar."""
    torch = _torch()
    ia = _lib()
    F, D, M = shape
    B, H, N = 2, 2, 37
    inp = W.make_inputs(B, H, N + 2, F, D, M, dtype="bf16", seed=F + 3 * D + 7 * M)
    lam, beta = inp["lam"], inp["beta"]
    q, k, v = (inp[n] for n in "qkv")
    bf = torch.bfloat16
    tag(f"bf16 prefill refused F={F} D={D} M={M}")
    st = ia.new_state(B, H, M, F, D)
    with pytest.raises(ia.IAError) as e:
        ia.prefill(dev(q[:, :N], bf), dev(k[:, :N], bf), dev(v[:, :N], bf), dev(lam), dev(beta),
                   state=st, out_dtype=torch.float32)
    assert e.value.status == 7
    tag(f"fp32 token-sequential prefill F={F} D={D} M={M}")
    o = ia.prefill(dev(q[:, :N]), dev(k[:, :N]), dev(v[:, :N]), dev(lam), dev(beta), state=st,
                   out_dtype=torch.float32)
    o_ref, _, _, st_ref = oracle.prefill(q[:, :N], k[:, :N], v[:, :N], lam, beta)
    torch.cuda.synchronize()
    err = rowrel(host(o), o_ref)
    report(f"token-sequential F={F} D={D} M={M} output", err)
    assert err < TOL_F32
    assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32
    st_ref = tuple(host(s) for s in st)   # both sides continue from the complex64 state
    for t in range(N, N + 2):
        tag(f"decode F={F} D={D} M={M} step {t - N}")
        o = ia.decode(dev(q[:, t], bf), dev(k[:, t], bf), dev(v[:, t], bf), dev(lam), dev(beta), st)
        o_ref, st_ref = oracle.decode_step(q[:, t], k[:, t], v[:, t], lam, beta, st_ref)
        torch.cuda.synchronize()
        assert rowrel(host(o), o_ref) < TOL_F32
        assert state_rel(tuple(host(s) for s in st), st_ref) < TOL_F32


@pytest.mark.parametrize("case", ["plain", "gated", "readout", "bidir"])
def test_fp32_prefill_segments_match_one_walk(case):
    """The register-resident walk cut into sequence segments (state-only pass from zero, the
    carry of the segment starts, every segment from its start; the workspace the query returns)
    against one walk of the whole sequence (a workspace too small for segments) and against
    the oracle: fp32 inputs, 4 slices of 700 tokens, a caller state (except bidirectional)."""
    torch = _torch()
    ia = _lib()
    B, H, N, F, D, M = 2, 2, 700, 64, 32, 16
    inp = W.make_inputs(B, H, N, F, D, M, dtype="f32", seed=40)
    q, k, v = (dev(inp[n]) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    rng = np.random.default_rng(41)
    kw, wg, dg, R = {}, None, None, None
    if case == "gated":
        wg = rng.uniform(0.0, 1.5, (B, N, H)).astype(np.float32)
        dg = rng.uniform(0.5, 1.0, (B, N, H)).astype(np.float32)
        kw["gates"] = (dev(wg), dev(dg))
    if case == "readout":
        X = rng.standard_normal((H, M, M)) + 1j * rng.standard_normal((H, M, M))
        R = (np.eye(M)[None] + 0.3 * X / np.sqrt(M)).astype(np.complex64)
        kw["readout"] = dev(R)
    bidir = case == "bidir"
    st0 = None
    if not bidir:
        pre = W.make_inputs(B, H, 9, F, D, M, dtype="f32", seed=42, std=0.5)
        st0 = tuple(host(dev(x)) for x in
                    oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3])
    one_walk = B * H * M * (F + D + 1) * 8 + 256   # a state: no room for segment slots
    runs = []
    for ws_bytes in (None, one_walk):
        tag(f"fp32 prefill segments {case} ws={ws_bytes}")
        st = None if bidir else tuple(dev(x) for x in st0)
        ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8,
                                                       device="cuda")
        o = ia.prefill(q, k, v, lam, beta, state=st, out_dtype=torch.float32, bidir=bidir,
                       workspace=ws, **kw)
        torch.cuda.synchronize()
        runs.append((host(o), None if st is None else tuple(host(x) for x in st)))
    (o_seg, s_seg), (o_one, s_one) = runs
    assert rowrel(o_seg, o_one) < 1e-4
    if not bidir:
        assert state_rel(s_seg, s_one) < 1e-4
    if case == "plain":
        o_ref, _, _, s_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"],
                                            inp["beta"], state=st0, threads=8)
    elif case == "gated":
        o_ref, _, _, s_ref = oracle.prefill_gated(inp["q"], inp["k"], inp["v"], inp["lam"],
                                                  inp["beta"], wg, dg, state=st0, threads=8)
    elif case == "readout":
        o_ref, _, _, s_ref = oracle.prefill_readout(inp["q"], inp["k"], inp["v"], inp["lam"],
                                                    inp["beta"], R, state=st0, threads=8)
    else:
        o_ref, s_ref = oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"],
                                    threads=8), None
    err = rowrel(o_seg, o_ref)
    report(f"fp32 prefill segments {case}", err)
    assert err < TOL_F32
    if s_ref is not None:
        assert state_rel(s_seg, s_ref) < TOL_F32
