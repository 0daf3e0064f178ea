"""GPU parity of the chunked MFMA prefill (bf16 inputs) against the oracle.

Every case compares every (b,h) slice, the full workload sizes included (in the launch
configuration the benchmark times), and the final state wherever the call returns one.
Tolerance: row-wise relative error 2e-2 (bf16 inputs).
"""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from helpers import TOL_BF16, dev, host, report, rowrel, state_rel, tag

pytestmark = pytest.mark.gpu


def _ia():
    import ssm_sequence_mixer_amd as ia
    return ia


def _run(inp, state=None, chunk=0, out="f32", bidir=False, want_output=True):
    import torch
    ia = _ia()
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    od = torch.float32 if out == "f32" else torch.bfloat16
    o = ia.prefill(q, k, v, dev(inp["lam"]), dev(inp["beta"]), state=state, out_dtype=od,
                   chunk=chunk, bidir=bidir, want_output=want_output)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("shape", [
    (2, 2, 200, 32, 16), (1, 3, 130, 64, 32), (1, 2, 257, 128, 64), (2, 1, 64, 32, 64),
    (1, 2, 1, 64, 16), (1, 1, 33, 128, 32)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_chunk_matches_oracle(shape, chunk):
    B, H, N, F, M = shape
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=100 + N + F + M + chunk)
    tag(f"chunk prefill B={B} H={H} N={N} F={F} M={M} C={chunk}")
    o = _run(inp, chunk=chunk)
    o_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])[0]
    err = rowrel(host(o), o_ref)
    report(f"chunk {shape} C={chunk}", err)
    assert err < TOL_BF16


@pytest.mark.parametrize("chunk", [32, 64])
def test_chunk_many_segments_with_state(chunk):
    """One sequence, 2048 tokens: the plan cuts it into many segments (carry scan), from a
    non-zero initial state; outputs and the final state against the oracle."""
    ia = _ia()
    B, H, N, F, M = 1, 1, 2048, 64, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=7 + chunk)
    pre = W.make_inputs(B, H, 20, F, F, M, dtype="bf16", seed=8)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"])[3]
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    tag(f"chunk prefill many segments C={chunk}")
    o = _run(inp, state=st, chunk=chunk)
    o_ref, _, _, st_out = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"],
                                         inp["beta"], state=st_ref)
    e_o, e_s = rowrel(host(o), o_ref), state_rel(tuple(host(s) for s in st), st_out)
    report(f"many segments C={chunk} output", e_o)
    report(f"many segments C={chunk} state", e_s)
    assert e_o < TOL_BF16 and e_s < TOL_BF16


def test_chunk_few_segments_with_state():
    """Many (b,h) slices, 2048 tokens, non-zero initial state: a few segments per sequence,
    whose output workgroups combine their predecessors' end states themselves."""
    B, H, N, F, M = 6, 16, 2048, 64, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=17)
    pre = W.make_inputs(B, H, 24, F, F, M, dtype="bf16", seed=18)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"], threads=8)[3]
    st = tuple(dev(s) for s in st_ref)
    st_ref = tuple(host(s) for s in st)
    tag("chunk prefill few segments with state")
    o = _run(inp, state=st)
    o_ref, _, _, st_out = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"],
                                         state=st_ref, threads=16)
    e_o = rowrel(host(o), o_ref)
    e_s = state_rel(tuple(host(s) for s in st), st_out)
    report("few segments output", e_o)
    report("few segments state", e_s)
    assert e_o < TOL_BF16 and e_s < TOL_BF16


def test_chunk_size_invariance():
    B, H, N, F, M = 2, 2, 300, 64, 64
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=55)
    tag("chunk size invariance")
    o32 = host(_run(inp, chunk=32))
    o64 = host(_run(inp, chunk=64))
    o_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])[0]
    e32, e64, e_x = rowrel(o32, o_ref), rowrel(o64, o_ref), rowrel(o32, o64)
    report("chunk 32 vs oracle", e32)
    report("chunk 64 vs oracle", e64)
    report("chunk 32 vs chunk 64", e_x)
    assert e32 < TOL_BF16 and e64 < TOL_BF16 and e_x < 2 * TOL_BF16


def test_state_only_prefill_then_decode():
    """State-only prefill (no outputs) then decode steps equal the full prefill's tail."""
    import torch
    ia = _ia()
    B, H, N, F, M = 2, 2, 150, 128, 64
    inp = W.make_inputs(B, H, N + 4, F, F, M, dtype="bf16", seed=77)
    head = {n: inp[n][:, :N] for n in "qkv"}
    head.update(lam=inp["lam"], beta=inp["beta"])
    st = ia.new_state(B, H, M, F, F)
    tag("state-only prefill")
    _run(head, state=st, want_output=False)
    outs = []
    for t in range(N, N + 4):
        outs.append(host(ia.decode(dev(inp["q"][:, t], torch.bfloat16),
                                   dev(inp["k"][:, t], torch.bfloat16),
                                   dev(inp["v"][:, t], torch.bfloat16), dev(inp["lam"]),
                                   dev(inp["beta"]), st)))
    torch.cuda.synchronize()
    o_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])[0]
    err = rowrel(np.stack(outs, axis=1), o_ref[:, N:])
    report("state-only prefill then decode", err)
    assert err < TOL_BF16


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_chunk_bidirectional(out):
    B, H, N, F, M = 1, 2, 333, 32, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=91)
    tag(f"chunk bidir out={out}")
    o = _run(inp, bidir=True, out=out)
    o_ref = oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
    err = rowrel(host(o), o_ref)
    report(f"chunk bidir out={out}", err)
    assert err < TOL_BF16


def test_chunk_forced_clamp():
    """beta = i with real lambda: Re(den) < 0 everywhere, o = num / clamp."""
    B, H, N, F, M = 1, 1, 100, 32, 16
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=13, dt=0.02,
                        beta=np.full((1, M), 1j))
    inp["lam"] = np.full((1, M), np.float32(0.95), np.complex64)
    tag("chunk forced clamp")
    o = _run(inp)
    o_ref, _, den, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
    assert np.all(den < 0)
    err = rowrel(host(o), o_ref)
    report("chunk forced clamp", err)
    assert err < TOL_BF16


@pytest.mark.parametrize("plan", [(1, 2, 1536), (4, 16, 512)])
def test_chunk_lambda_edges_multi_segment(plan):
    """Modes on and near the unit circle among the S4D modes, several segments per sequence:
    (1, 2, 1536) runs many segments through the carry kernel, (4, 16, 512) four segments
    through the Horner step; outputs and the final state in every case, beta = 1.

    - near one (lam = 1, exp(-1e-6 + 1e-6 i)): the chunked path (its segment end states take
      the powers of lam by binary exponentiation and sum_n beta lam^n in closed form);
    - damped large arguments (exp(-0.01 - 3.1 i), exp(-0.003 + 2.5 i), 0.995 e^(0.9 i pi),
      |1 - lam|^2 / (1 - |lam|^2) from 200 to 900): the chunked path;
    - undamped large arguments (-1, i, 0.999 e^(0.999 i pi)): every head holds one, so every
      head runs the fp32 route inside the chunked launches, at the fp32 tolerance (the inputs
      are bf16-exact, the oracle sees the same values).
    ia_check_lambda's count of routed heads is checked against each case.  (A head without
    a slow non-rotating mode, e.g. with these modes in place of mode 0, has Re(den) negative
    in most rows and cancelling in the rest: ill-conditioned for any precision, and beyond
    what bf16 operands resolve.)"""
    import torch
    ia = _ia()
    from helpers import TOL_F32
    B, H, N = plan
    F, M = 64, 32
    cases = [
        ("near one", [1.0, np.exp(-1e-6 + 1e-6j)], False),
        ("damped large argument", [np.exp(-0.01 - 3.1j), np.exp(-0.003 + 2.5j),
                                   0.995 * np.exp(0.9j * np.pi)], False),
        ("undamped large argument", [-1.0, 1j, 0.999 * np.exp(1j * np.pi * 0.999)], True)]
    for name, edge, routed in cases:
        edge = np.array(edge, np.complex64)
        inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=301 + N)
        lam = inp["lam"].copy()
        # near one: in place of the slowest modes; the others among the fast ones, next to
        # mode 0 (exp(-dt/2), real), whose large positive eta keeps Re(den) well conditioned
        at = slice(0, len(edge)) if name == "near one" else slice(M - len(edge), M)
        for h in range(H):
            lam[h, at] = np.roll(edge, h)
        inp["lam"] = lam
        desc = ia.make_desc(B, H, N, F, F, M)
        assert ia.ia_check_lambda(desc, lam) == (H if routed else 0)
        st = ia.new_state(B, H, M, F, F)
        tag(f"chunk lambda edges ({name}) B={B} H={H} N={N}")
        o = _run(inp, state=st)
        o_ref, _, _, st_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"],
                                             inp["beta"], threads=8)
        tol = TOL_F32 if routed else TOL_BF16
        e_s = state_rel(tuple(host(s) for s in st), st_ref)
        e_o = rowrel(host(o), o_ref)
        report(f"lambda edges ({name}) {plan} state", e_s)
        report(f"lambda edges ({name}) {plan} output", e_o)
        assert e_s < tol and e_o < tol


@pytest.mark.parametrize("kind", ["fast", "undamped"])
@pytest.mark.parametrize("mode", ["state", "several segments", "no state", "state only",
                                  "bidirectional"])
def test_fp32_route_heads(kind, mode):
    """Heads the chunk factorisation does not resolve run the fp32 recurrence inside the
    chunked launches, next to heads that take the chunked path: "fast" gives head 1 S4D-Lin
    modes at dt = 0.3 (|lam|^63 < 2^-8), "undamped" gives head 1 a mode at -1.  Head 0 stays
    chunked.  Each call form: with a caller state (one segment: 16 slices fill the device
    with G = 1 only when N is short, so the plan varies), with a state and several segments
    (the initial state read from its workspace copy), without a state (the route's working
    state in the workspace), state only, and bidirectional (both walks on the route)."""
    import torch
    ia = _ia()
    from helpers import TOL_F32
    B, H, F, M = 2, 2, 64, 32
    N = 700 if mode != "state" else 64
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=611 + N)
    lam = inp["lam"].copy()
    if kind == "fast":
        lam[1] = W.s4d_lin(np.array([0.3]), M)[0]
    else:
        lam[1, 7] = -1.0
    inp["lam"] = lam
    assert ia.ia_check_lambda(ia.make_desc(B, H, N, F, F, M), lam) == 1
    tag(f"fp32 route ({kind}, {mode}) B={B} H={H} N={N}")
    if mode == "bidirectional":
        o = host(_run(inp, bidir=True))
        ref = oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"])
        e0, e1 = rowrel(o[:, :, 0], ref[:, :, 0]), rowrel(o[:, :, 1], ref[:, :, 1])
        report(f"fp32 route ({kind}, {mode}) chunked head / routed head", max(e0, e1))
        assert e0 < TOL_BF16 and e1 < TOL_F32
        return
    st = None
    st_ref0 = None
    if mode in ("state", "several segments", "state only"):
        pre = W.make_inputs(B, H, 10, F, F, M, dtype="bf16", seed=612)
        st_ref0 = oracle.prefill(pre["q"], pre["k"], pre["v"], lam, inp["beta"])[3]
        st = tuple(dev(x) for x in st_ref0)
        st_ref0 = tuple(host(x) for x in st)
    o = _run(inp, state=st, want_output=mode != "state only")
    o_ref, _, _, st_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], lam, inp["beta"],
                                         state=st_ref0)
    if o is not None:
        o = host(o)
        e0, e1 = rowrel(o[:, :, 0], o_ref[:, :, 0]), rowrel(o[:, :, 1], o_ref[:, :, 1])
        report(f"fp32 route ({kind}, {mode}) outputs chunked head / routed head", max(e0, e1))
        assert e0 < TOL_BF16 and e1 < TOL_F32
    if st is not None:
        got = tuple(host(x) for x in st)
        e0 = state_rel(tuple(x[:, :1] for x in got), tuple(x[:, :1] for x in st_ref))
        e1 = state_rel(tuple(x[:, 1:] for x in got), tuple(x[:, 1:] for x in st_ref))
        report(f"fp32 route ({kind}, {mode}) states chunked head / routed head", max(e0, e1))
        assert e0 < TOL_BF16 and e1 < TOL_F32


# ---------------------------------------------------------------- full workload sizes
# Every (b, h) slice at the full sizes, in the launch configuration the benchmark times; the
# causal runs pass a zero initial state so the final state is returned and compared too.
# The worst slice is printed with its head (the smallest-dt heads carry the largest bf16
# error: their modes remember the most tokens).

def _worst_slice(o, ref):
    B, H = o.shape[0], o.shape[2]
    errs = np.array([[rowrel(o[b, :, h], ref[b, :, h]) for h in range(H)] for b in range(B)])
    b, h = np.unravel_index(np.argmax(errs), errs.shape)
    return float(errs[b, h]), (int(b), int(h)), errs.max(axis=0)


def _full(inp, out="f32", with_state=True, threads=16, ref=None):
    ia = _ia()
    sh = inp["shape"]
    B, H, F, D, M = sh["B"], sh["H"], sh["F"], sh["D"], sh["M"]
    st = ia.new_state(B, H, M, F, D) if with_state else None
    o = host(_run(inp, state=st, out=out))
    if ref is None:
        ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"],
                             threads=threads)
    o_ref, _, _, st_ref = ref
    worst, where, per_head = _worst_slice(o, o_ref)
    e_s = state_rel(tuple(host(s) for s in st), st_ref) if with_state else 0.0
    return worst, where, e_s, per_head


def _check_full(name, inp, res):
    worst, where, e_s, per_head = res
    dt = np.asarray(inp["dt"])
    report(f"{name} output (worst slice b,h={where}, dt={dt[where[1]]:.2e})", worst)
    report(f"{name} final state", e_s)
    print(f"[err] {name} per head: " + " ".join(f"h{h}:{e:.1e}" for h, e in enumerate(per_head)),
          flush=True)
    assert worst < TOL_BF16 and e_s < TOL_BF16


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_workload_125m_all_slices(out):
    inp = W.l125m()
    tag(f"125m workload out={out}, every slice and the final state")
    _check_full(f"125m out={out}", inp, _full(inp, out=out))


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_workload_1p3b_all_slices(out):
    inp = W.l1p3b()
    tag(f"1.3b workload out={out}, every slice and the final state")
    _check_full(f"1.3b out={out}", inp, _full(inp, out=out))


def test_workload_1p3b_long_all_slices():
    inp = W.l1p3b(N=7168)
    tag("1.3b x3.5 length workload, every slice and the final state")
    _check_full("1.3b x3.5 length", inp, _full(inp, out="bf16"))


def test_workload_caduceus_all_slices():
    """The genomic workload on every (b, h) slice: the bidirectional layer as the benchmark
    runs it (bf16 out, both directions summed), then each direction alone as a causal run with
    its final state (the forward sequence, and the flipped sequence for the reverse
    direction).  The oracle's two directions serve all three comparisons."""
    inp = W.caduceus()
    fl = dict(inp)
    for n in "qkv":
        fl[n] = np.ascontiguousarray(inp[n][:, ::-1])
    ref_f = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"], threads=16)
    ref_r = oracle.prefill(fl["q"], fl["k"], fl["v"], inp["lam"], inp["beta"], threads=16)
    tag("caduceus bidirectional workload, every slice")
    o = host(_run(inp, bidir=True, out="bf16"))
    worst, where, per_head = _worst_slice(o, ref_f[0] + ref_r[0][:, ::-1])
    del o
    report(f"caduceus bidir (worst slice b,h={where}, dt={inp['dt'][where[1]]:.2e})", worst)
    print("[err] caduceus bidir per head: " +
          " ".join(f"h{h}:{e:.1e}" for h, e in enumerate(per_head)), flush=True)
    assert worst < TOL_BF16
    tag("caduceus forward direction, causal with state")
    _check_full("caduceus forward", inp, _full(inp, out="bf16", ref=ref_f))
    tag("caduceus reverse direction, causal with state")
    _check_full("caduceus reverse", fl, _full(fl, out="bf16", ref=ref_r))


# ---------------------------------------------------------------- strided inputs

def _state_from(inp, B, H, F, M, seed):
    pre = W.make_inputs(B, H, 12, F, F, M, dtype="bf16", seed=seed)
    st_ref = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"], threads=8)[3]
    return st_ref


@pytest.mark.parametrize("plan", [(1, 2, 700, 64, 32), (4, 16, 512, 128, 64)])
@pytest.mark.parametrize("layout", ["qkv fused", "qk fused, v wide"])
def test_chunk_strided_inputs(plan, layout):
    """q, k, v as views (ia_prefill_fwd_strided): "qkv fused" slices one [B][N][3][H][F]
    projection; "qk fused, v wide" slices q, k from [B][N][2][H][F] and v from the first half
    of a [B][N][H][2F] tensor (v strides differ from q's).  With an initial state, several
    segments ((1, 2, 700): carry; (4, 16, 512): Horner).  The strided call equals the dense
    call on contiguous copies exactly, and the oracle within the bf16 tolerance."""
    import torch
    ia = _ia()
    B, H, N, F, M = plan
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=401 + N + F)
    q0, k0, v0 = (dev(inp[n], torch.bfloat16) for n in "qkv")
    if layout == "qkv fused":
        fused = torch.stack([q0, k0, v0], dim=2)                  # [B, N, 3, H, F]
        q, k, v = fused[:, :, 0], fused[:, :, 1], fused[:, :, 2]
    else:
        fused = torch.stack([q0, k0], dim=2)                      # [B, N, 2, H, F]
        q, k = fused[:, :, 0], fused[:, :, 1]
        wide = torch.cat([v0, torch.zeros_like(v0)], dim=3)      # [B, N, H, 2F]
        v = wide[..., :F]
    assert not (q.is_contiguous() or k.is_contiguous() or v.is_contiguous())
    st_ref = _state_from(inp, B, H, F, M, seed=402)
    st_s = tuple(dev(s) for s in st_ref)
    st_d = tuple(dev(s) for s in st_ref)
    st_in = tuple(host(s) for s in st_s)
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    tag(f"strided prefill ({layout}) B={B} H={H} N={N} F={F} M={M}")
    o_s = ia.prefill(q, k, v, lam, beta, state=st_s, out_dtype=torch.float32)
    o_d = ia.prefill(q0, k0, v0, lam, beta, state=st_d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d)
    assert all(torch.equal(a, b) for a, b in zip(st_s, st_d))
    o_ref, _, _, st_out = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"],
                                         state=st_in, threads=8)
    e_o = rowrel(host(o_s), o_ref)
    e_s = state_rel(tuple(host(s) for s in st_s), st_out)
    report(f"strided ({layout}) {plan} output", e_o)
    report(f"strided ({layout}) {plan} state", e_s)
    assert e_o < TOL_BF16 and e_s < TOL_BF16


def test_strided_inputs_bidirectional_and_fp32():
    """Strided views through the reverse walk (bidirectional, bf16) and through the
    token-sequential fp32 path: equal to the dense calls, near the oracle."""
    import torch
    from helpers import TOL_F32
    ia = _ia()
    B, H, N, F, M = 1, 3, 333, 32, 32
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=91)
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    q0, k0, v0 = (dev(inp[n], torch.bfloat16) for n in "qkv")
    fused = torch.stack([q0, k0, v0], dim=2)
    tag("strided bidirectional")
    o_s = ia.prefill(fused[:, :, 0], fused[:, :, 1], fused[:, :, 2], lam, beta, bidir=True,
                     out_dtype=torch.float32)
    o_d = ia.prefill(q0, k0, v0, lam, beta, bidir=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d)
    err = rowrel(host(o_s), oracle.bidir(inp["q"], inp["k"], inp["v"], inp["lam"], inp["beta"]))
    report("strided bidir", err)
    assert err < TOL_BF16

    inp = W.make_inputs(1, 2, 150, 32, 32, 16, dtype="f32", seed=92)
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    q0, k0, v0 = (dev(inp[n]) for n in "qkv")
    fused = torch.stack([q0, k0, v0], dim=2)
    tag("strided fp32 prefill")
    o_s = ia.prefill(fused[:, :, 0], fused[:, :, 1], fused[:, :, 2], lam, beta)
    o_d = ia.prefill(q0, k0, v0, lam, beta)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d)
    err = rowrel(host(o_s), oracle.prefill(inp["q"], inp["k"], inp["v"], inp["lam"],
                                           inp["beta"])[0])
    report("strided fp32", err)
    assert err < TOL_F32
