"""C ABI of libia.so, host side only (no GPU): exports and every validation path.

Each call here fails validation, which the library finishes before it enqueues anything,
so the fake device addresses below are never dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import ssm_sequence_mixer_amd as ia

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ia.h")
P = ctypes.c_void_p
BASE = 1 << 32            # fake, 16-byte aligned device addresses, far apart
GAP = 1 << 28


def addr(i, off=0):
    return P(BASE + i * GAP + off)


def desc(**kw):
    d = dict(B=2, H=3, N=70, F=32, Dv=16, M=16, in_dtype=ia.IA_BF16, out_dtype=ia.IA_F32,
             den_clamp=1e-6, bidir=False, chunk=0)
    d.update(kw)
    return ia.make_desc(**d)


def _has_device():
    import torch
    return torch.cuda.device_count() > 0


def state(i=10):
    return ctypes.pointer(ia.IAState(addr(i).value, addr(i + 1).value, addr(i + 2).value))


def prefill(d, q=None, k=None, v=None, lam=None, beta=None, st="default", o=None, ws=None,
            ws_bytes=1 << 40):
    q = addr(0) if q is None else q
    k = addr(1) if k is None else k
    v = addr(2) if v is None else v
    lam = addr(3) if lam is None else lam
    beta = addr(4) if beta is None else beta
    st = state() if isinstance(st, str) else st
    o = addr(5) if o is None else o
    ws = addr(6) if ws is None else ws
    return ia.lib.ia_prefill_fwd(ctypes.byref(d) if d is not None else None, q, k, v, lam, beta,
                                 st, o, ws, ws_bytes, None)


def test_every_declared_symbol_is_exported():
    decl = set(re.findall(r"^\s*(?:ia_status|size_t|const char\*)\s+(ia_\w+)\s*\(",
                          open(HEADER).read(), flags=re.M))
    assert decl == set(ia.EXPORTS)
    for name in decl:
        assert hasattr(ia.lib, name), name


def test_status_strings():
    for code, name in enumerate(ia.STATUS):
        assert ia.lib.ia_status_string(code).decode().startswith(name)


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, 2), ("H", -1, 2), ("N", 0, 2), ("F", 0, 2), ("Dv", 0, 2), ("M", 0, 2),
    ("F", 24, 7), ("Dv", 8, 7), ("M", 20, 7), ("F", 272, 7), ("Dv", 512, 7), ("M", 144, 7),
    ("in_dtype", 2, 3), ("out_dtype", -1, 3),
    ("den_clamp", 0.0, 6), ("den_clamp", -1e-6, 6), ("den_clamp", float("nan"), 6),
    ("den_clamp", float("inf"), 6), ("chunk", 48, 7), ("chunk", 16, 7)])
def test_desc_validation(field, value, status):
    d = desc()
    setattr(d, field, value)
    assert prefill(d) == status
    if field not in ("N",):
        assert ia.lib.ia_decode_step(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3),
                                     addr(4), state(), addr(5), None) == status
        assert ia.lib.ia_state_init(ctypes.byref(d), state(), None) == status
    assert ia.lib.ia_prefill_workspace_bytes(ctypes.byref(d)) == 0


def test_unknown_flag_bits():
    for bits in (32, 64, 1 << 31, 1 | 32):
        d = desc()
        d.flags = bits
        assert prefill(d) == 7, bits


def test_known_flag_combinations_accepted_by_validation():
    # Bits 1 to 16 are defined: every combination passes the flag check (the call then fails
    # on the bad shape, not on the flags).
    for bits in range(32):
        d = desc()
        d.flags = bits
        d.N = 0
        assert prefill(d) == 2, bits


def test_null_pointers():
    assert prefill(None) == 1
    for kw in ("q", "k", "v", "lam", "beta"):
        assert prefill(desc(), **{kw: P(0)}) == 1, kw
    # o and state both absent: nothing to compute
    assert prefill(desc(), st=None, o=P(0)) == 1
    assert prefill(desc(), st=ctypes.pointer(ia.IAState(addr(10).value, 0, addr(12).value))) == 1
    assert ia.lib.ia_state_init(ctypes.byref(desc()), None, None) == 1
    assert ia.lib.ia_decode_step(ctypes.byref(desc()), addr(0), addr(1), addr(2), addr(3),
                                 addr(4), None, addr(5), None) == 1
    assert ia.lib.ia_decode_step(ctypes.byref(desc()), addr(0), addr(1), addr(2), addr(3),
                                 addr(4), state(), P(0), None) == 1


def test_alignment():
    for kw in ("q", "k", "v", "lam", "beta", "o"):
        assert prefill(desc(), **{kw: addr({"q": 0, "k": 1, "v": 2, "lam": 3, "beta": 4,
                                            "o": 5}[kw], 8)}) == 4, kw
    bad = ctypes.pointer(ia.IAState(addr(10, 4).value, addr(11).value, addr(12).value))
    assert prefill(desc(), st=bad) == 4
    assert ia.lib.ia_state_init(ctypes.byref(desc()), bad, None) == 4


def test_aliasing():
    d = desc()
    # o overlapping each input, and the state
    for i in range(5):
        assert prefill(d, o=addr(i, 16)) == 5, i
    assert prefill(d, o=addr(10, 32)) == 5
    # state overlapping an input
    st = ctypes.pointer(ia.IAState(addr(0, 64).value, addr(11).value, addr(12).value))
    assert prefill(d, st=st) == 5
    # state buffers overlapping each other
    st = ctypes.pointer(ia.IAState(addr(10).value, addr(10, 256).value, addr(12).value))
    assert prefill(d, st=st) == 5
    # decode: o_t overlapping the state
    assert ia.lib.ia_decode_step(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3), addr(4),
                                 state(), addr(11, 16), None) == 5


def test_bidir_rules():
    d = desc(bidir=True)
    assert prefill(d) == 7                    # a state with BIDIR
    assert prefill(d, st=None, o=P(0)) == 1   # BIDIR needs an output
    assert ia.lib.ia_decode_step(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3), addr(4),
                                 state(), addr(5), None) == 7


def test_workspace_checks():
    for in_dtype in (ia.IA_F32, ia.IA_BF16):
        d = desc(in_dtype=in_dtype, Dv=32)
        need = ia.lib.ia_prefill_workspace_bytes(ctypes.byref(d))
        assert need > 0
        assert prefill(d, st=None, ws=P(0)) == 9
        assert prefill(d, st=None, ws_bytes=need - 1) == 9
        # workspace overlapping an input
        assert prefill(d, st=None, ws=addr(1, 32)) in (5,)


@pytest.mark.parametrize("shape", [dict(F=32, Dv=16), dict(F=64, Dv=128), dict(F=256, Dv=256),
                                   dict(F=128, Dv=128, M=128), dict(F=16, Dv=16)])
def test_bf16_shapes_without_chunk_kernel_are_refused(shape):
    """bf16 inputs take the chunked MFMA kernels only (F = Dv in {32, 64, 128}, M <= 64); any
    other bf16 shape is refused, not run by the token-sequential kernel, and has no workspace
    size.  The same shapes in fp32 are accepted by validation (they reach the workspace
    check here)."""
    d = desc(**shape)
    assert ia.lib.ia_prefill_workspace_bytes(ctypes.byref(d)) == 0
    assert prefill(d) == 7
    assert prefill_strided(d, None) == 7
    f = desc(in_dtype=ia.IA_F32, **shape)
    assert ia.lib.ia_prefill_workspace_bytes(ctypes.byref(f)) > 0
    assert prefill(f, st=None, ws=P(0)) == 9


def test_bf16_rows_beyond_32bit_offsets_are_refused():
    # 64 token rows of H*F bf16 values must span at most 1 GiB for the chunk kernels
    d = desc(H=65540, F=128, Dv=128, M=16, B=1, N=1)
    assert prefill(d, st=None) == 7


def s4d(dt, M):
    return np.exp(dt * (-0.5 + 1j * np.pi * np.arange(M))).astype(np.complex64)


def test_check_lambda_host():
    """IA_ERR_DOMAIN outside 0 < |lambda| <= 1 + 1e-6; the count of heads the chunked bf16
    prefill runs on its fp32 route (the same test the device applies to its tables)."""
    d = desc(H=1, M=16)
    assert ia.ia_check_lambda(d, s4d(0.05, 16)[None]) == 0
    for bad in (np.zeros(16), 1.1 * np.ones(16), np.full(16, np.nan)):
        with pytest.raises(ia.IAError) as e:
            ia.ia_check_lambda(d, bad.astype(np.complex64)[None])
        assert e.value.status == 6
    # a fast mode: |lambda|^63 < 2^-8 at chunk 64, not at chunk 32 (0.9^31 = 0.038)
    mid = (0.9 * np.ones(16, np.complex64))[None]
    assert ia.ia_check_lambda(desc(H=1, M=16), mid) == 1
    assert ia.ia_check_lambda(desc(H=1, M=16, chunk=32), mid) == 0
    # fp32 inputs never take the chunked path
    assert ia.ia_check_lambda(desc(H=1, M=16, in_dtype=ia.IA_F32), (0.5 * mid)) == 0
    # undamped modes: lambda = 1 (and next to it) stays, -1, i and 0.999 e^(0.999 i pi) route
    near = s4d(0.05, 16)
    near[:2] = [1.0, np.exp(-1e-6 + 1e-6j)]
    assert ia.ia_check_lambda(d, near[None]) == 0
    for edge in (-1.0, 1j, 0.999 * np.exp(1j * np.pi * 0.999)):
        lam = s4d(0.05, 16)
        lam[3] = edge
        assert ia.ia_check_lambda(d, lam[None]) == 1, edge
    # damped enough: exp(-0.01 - 3.1 i) has |1 - lam|^2 / (1 - |lam|^2) of about 200
    lam = s4d(0.05, 16)
    lam[3] = np.exp(-0.01 - 3.1j)
    assert ia.ia_check_lambda(d, lam[None]) == 0
    # S4D-Lin modes stay on the chunked path (M = 64) for every dt up to 0.17, past the
    # workloads' range [1e-3, 1e-1]; beyond, |lambda|^63 < 2^-8 routes them
    dts = np.exp(np.linspace(np.log(1e-4), np.log(0.17), 41))
    assert ia.ia_check_lambda(desc(H=41, M=64), np.stack([s4d(t, 64) for t in dts])) == 0
    assert ia.ia_check_lambda(desc(H=1, M=64), s4d(0.2, 64)[None]) == 1
    # heads are counted one by one
    two = np.stack([s4d(0.01, 16), s4d(0.01, 16)])
    two[1, 5] = -1.0
    assert ia.ia_check_lambda(desc(H=2, M=16), two) == 1


def prefill_strided(d, strides, **kw):
    """ia_prefill_fwd_strided with the fake addresses of prefill(); strides = 3 (b, n, h)
    triples for q, k, v, or None."""
    st = None
    if strides is not None:
        st = ((ctypes.c_longlong * 3) * 3)()
        for i in range(3):
            for j in range(3):
                st[i][j] = strides[i][j]
    a = dict(q=addr(0), k=addr(1), v=addr(2), lam=addr(3), beta=addr(4), st=state(), o=addr(5),
             ws=addr(6), ws_bytes=1 << 40)
    a.update(kw)
    return ia.lib.ia_prefill_fwd_strided(ctypes.byref(d), a["q"], a["k"], a["v"],
                                         ctypes.byref(st) if st is not None else None,
                                         a["lam"], a["beta"], a["st"], a["o"], a["ws"],
                                         a["ws_bytes"], None)


def test_strided_validation():
    """Each case fails validation (nothing is launched on the fake addresses)."""
    d = desc()                                   # B=2, H=3, N=70, F=32, Dv=16, bf16 inputs
    qk, vv = (70 * 3 * 32, 3 * 32, 32), (70 * 3 * 16, 3 * 16, 16)
    fused = (70 * 3 * 96, 3 * 96, 32)            # views of a [B][N][3][H][F] projection
    # the dense strides pass validation as ia_prefill_fwd does: same errors as there
    assert prefill_strided(d, [qk, qk, vv], q=P(0)) == 1
    assert prefill_strided(d, None, q=P(0)) == 1
    assert prefill_strided(d, [fused, fused, vv], o=addr(5, 8)) == 4
    # a stride <= 0
    for i in range(3):
        for j in range(3):
            bad = [list(qk), list(qk), list(vv)]
            bad[i][j] = 0 if j else -bad[i][j]
            if i < 2:
                bad[1 - i][j] = bad[i][j]        # keep q and k equal
            assert prefill_strided(d, bad) == 2, (i, j)
    # a stride whose byte size is not a multiple of 16 (bf16: 8 elements)
    assert prefill_strided(d, [(qk[0], qk[1], 36), (qk[0], qk[1], 36), vv]) == 4
    assert prefill_strided(d, [qk, qk, (vv[0], 52, vv[2])]) == 4
    # q and k with different strides
    assert prefill_strided(d, [qk, fused, vv]) == 7
    # 64 token rows spanning more than 1 GiB (bf16 chunk path, which needs F = Dv)
    d2 = desc(Dv=32)
    big = (1 << 24) + 8
    assert prefill_strided(d2, [(70 * big, big, 32), (70 * big, big, 32), qk]) == 7
    assert prefill_strided(d2, [qk, qk, (70 * big, big, 32)]) == 7
    # an input's strided extent reaching o (v's batch stride spans three address gaps)
    far = (3 * GAP) // 2 + 64
    assert prefill_strided(d, [qk, qk, (far, vv[1], vv[2])]) == 5


# ---------------------------------------------------------------- ia_prefill_bwd

def bwd(d, ws_bytes=1 << 40, st0=None, dst0=None, **ptrs):
    p = dict(q=addr(0), k=addr(1), v=addr(2), lam=addr(3), beta=addr(4), dO=addr(5),
             dq=addr(6), dk=addr(7), dv=addr(8), dlam=addr(9), dbeta=addr(13), ws=addr(14))
    p.update(ptrs)
    return ia.lib.ia_prefill_bwd(ctypes.byref(d) if d is not None else None, p["q"], p["k"],
                                 p["v"], p["lam"], p["beta"], st0, p["dO"], p["dq"], p["dk"],
                                 p["dv"], p["dlam"], p["dbeta"], dst0, p["ws"], ws_bytes, None)


def _bwd_chunked_bytes(B, H, N, F, D, M):
    """Workspace of the chunked backward (F == Dv in {32, 64, 128}): every 16-token chunk's
    start state per group of 16 modes (Re and Im rows of U, Gamma, eta, fp32), the per-token
    den and g.num partials per group, the groups' gradient rows, the lambda/beta partials."""
    up = lambda x: (x + 255) // 256 * 256
    S, G, nch = B * H, M // 16, (N + 15) // 16
    return (up(S * G * nch * 32 * (F + D + 1) * 4) + up(S * N * G * 8)
            + up(G * S * N * (2 * F + D) * 4) + up(S * M * 16))


def test_bwd_workspace_bytes_layout():
    up = lambda x: (x + 255) // 256 * 256
    for B, H, N, F, D, M in ((2, 3, 70, 32, 16, 16), (4, 16, 2048, 128, 128, 64),
                             (1, 1, 1, 16, 256, 128), (2, 8, 131072, 32, 32, 32),
                             (1, 2, 1000, 32, 32, 16)):
        chunked = F == D and F in (32, 64, 128)
        if chunked:
            d = desc(B=B, H=H, N=N, F=F, Dv=D, M=M)
            d.flags = ia.IA_FLAG_CHUNKED_BWD
            assert (ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d))
                    == _bwd_chunked_bytes(B, H, N, F, D, M))
        S, nck = B * H, (N + 31) // 32
        # sequence segments of the backward sweeps (no device: 256 compute units)
        wgs = S * (M // 16)
        n = 1 if wgs >= 256 else 256 // wgs
        n = max(1, min(n, (N + 255) // 256))
        seg = ((N + n - 1) // n + 31) // 32 * 32
        nseg = (N + seg - 1) // seg
        carry = up(S * nseg * M * (F + D + 1) * 8) if nseg > 1 else 0
        want = (up(S * nck * M * (F + D + 1) * 8) + up(S * N * (M // 2) * 8)
                + up((M // 16) * S * N * (2 * F + D) * 4) + up(S * nseg * M * 16)
                + up(S * N * M * 8) + 2 * carry)
        d = desc(B=B, H=H, N=N, F=F, Dv=D, M=M)
        d.flags = ia.IA_FLAG_SEQUENTIAL_BWD   # the token-sequential kernels' layout
        assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) == want
        if not chunked:
            d.flags = 0
            assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) == want
    assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(desc(N=0))) == 0
    assert ia.lib.ia_prefill_bwd_workspace_bytes(None) == 0
    # automatic choice: few slices and a long sequence take the token-sequential sweeps (cut
    # into more than eight segments), more slices the chunked kernels; the chunked flag forces
    # the chunked kernels' layout
    d = desc(B=1, H=2, N=4000, F=32, Dv=32, M=16)
    assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) != _bwd_chunked_bytes(
        1, 2, 4000, 32, 32, 16)
    d.flags = ia.IA_FLAG_CHUNKED_BWD
    assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) == _bwd_chunked_bytes(
        1, 2, 4000, 32, 32, 16)
    d = desc(B=2, H=8, N=131072, F=32, Dv=32, M=32)
    assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) == _bwd_chunked_bytes(
        2, 8, 131072, 32, 32, 32)
    # the chunked kernels exist for F == Dv in {32, 64, 128} only; both flags: unsupported
    d = desc(B=1, H=1, N=10, F=64, Dv=32, M=16)
    d.flags = ia.IA_FLAG_CHUNKED_BWD
    assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) == 0
    d = desc(B=1, H=1, N=10, F=32, Dv=32, M=16)
    d.flags = ia.IA_FLAG_CHUNKED_BWD | ia.IA_FLAG_SEQUENTIAL_BWD
    assert ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d)) == 0


def test_bwd_validation():
    d = desc()
    assert bwd(None) == 1
    assert bwd(desc(N=0)) == 2
    assert bwd(desc(M=20)) == 7
    dc = desc(Dv=48)
    dc.flags = ia.IA_FLAG_CHUNKED_BWD
    assert bwd(dc) == 7
    assert bwd(desc(bidir=True), st0=state()) == 7
    assert bwd(desc(bidir=True), dst0=state(20)) == 7
    for name in ("q", "k", "v", "lam", "beta", "dO", "dq", "dk", "dv", "dlam", "dbeta"):
        assert bwd(d, **{name: P(0)}) == 1, name
        assert bwd(d, **{name: addr(["q", "k", "v", "lam", "beta", "dO", "dq", "dk", "dv",
                                     "dlam", "dbeta"].index(name), 8)}) == 4, name
    need = ia.lib.ia_prefill_bwd_workspace_bytes(ctypes.byref(d))
    assert bwd(d, ws=P(0)) == 9
    assert bwd(d, ws_bytes=need - 1) == 9
    assert bwd(d, ws=addr(14, 8)) == 4
    # outputs overlapping inputs, each other or the workspace
    assert bwd(d, dq=addr(0)) == 5
    assert bwd(d, dv=addr(5)) == 5
    assert bwd(d, dk=addr(6, 64)) == 5
    assert bwd(d, dlam=addr(14, 256)) == 5
    # a state with a missing tensor, and a state gradient overlapping an input
    assert bwd(d, st0=ctypes.pointer(ia.IAState(addr(10).value, addr(11).value, 0))) == 1
    assert bwd(d, dst0=ctypes.pointer(ia.IAState(addr(0).value, addr(11).value,
                                                 addr(12).value))) == 5


def test_readout_variants_validation():
    d = desc()
    rd = addr(20)
    assert ia.lib.ia_prefill_fwd_readout(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3),
                                         addr(4), None, state(), addr(5), addr(6), 1 << 40,
                                         None) == 1
    assert ia.lib.ia_prefill_fwd_readout(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3),
                                         addr(4), addr(20, 8), state(), addr(5), addr(6),
                                         1 << 40, None) == 4
    # readout overlapping the output
    assert ia.lib.ia_prefill_fwd_readout(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3),
                                         addr(4), addr(5), state(), addr(5, 256), addr(6),
                                         1 << 40, None) == 5
    assert ia.lib.ia_decode_step_readout(ctypes.byref(d), addr(0), addr(1), addr(2), addr(3),
                                         addr(4), None, state(), addr(5), None) == 1
    assert ia.lib.ia_decode_step_readout(ctypes.byref(desc(bidir=True)), addr(0), addr(1),
                                         addr(2), addr(3), addr(4), rd, state(), addr(5),
                                         None) == 7
    # readout workspace: one state, rounded up to 256 bytes
    B, H, M, F, D = 2, 3, 16, 32, 16
    want = (B * H * M * (F + D + 1) * 8 + 255) // 256 * 256
    assert ia.lib.ia_prefill_readout_workspace_bytes(ctypes.byref(d)) == want
    # bf16 chunk shapes take the chunked path: its plan plus each head's readout-matrix
    # operand (fp16 2M x 2M and its scale, 256-byte aligned).  Without a device the plans
    # assume one workgroup per CU either way.
    dc = desc(F=64, Dv=64, M=64)
    extra = (3 * ((8 * 64 * 64 + 4 + 255) // 256 * 256) + 255) // 256 * 256
    if not _has_device():
        assert (ia.lib.ia_prefill_readout_workspace_bytes(ctypes.byref(dc))
                == ia.lib.ia_prefill_workspace_bytes(ctypes.byref(dc)) + extra)
    # F = Dv = 128 with M = 64: no 64-token readout-matrix instantiation
    big = desc(F=128, Dv=128, M=64, chunk=64)
    assert ia.lib.ia_prefill_fwd_readout(ctypes.byref(big), addr(0), addr(1), addr(2), addr(3),
                                         addr(4), rd, state(), addr(5), addr(6), 1 << 40,
                                         None) == 7


def test_block_edges_validation():
    d = desc(Dv=32)   # B=2, H=3, N=70, F=32, Dv=32
    W = 4

    def params(**kw):
        p = dict(conv_width=W, conv_q=addr(20).value, conv_k=addr(21).value,
                 conv_v=addr(22).value, rope_base=1e4, pos0=0, norm_gain=addr(23).value,
                 norm_bias=addr(24).value, norm_eps=1e-6)
        p.update(kw)
        return ia.IABlockParams(**p)

    def pro(p=None, d=d, q=0, st_in=None, st_out=None, fq=5, fk=6, vo=7):
        return ia.lib.ia_block_prologue(
            ctypes.byref(d), None if p is False else ctypes.byref(p or params()),
            None if q is None else addr(q),
            addr(1), addr(2), st_in, st_out, addr(fq), addr(fk), addr(vo), None)
    assert pro(False) == 1
    assert pro(params(conv_width=9)) == 7
    assert pro(params(conv_width=-1)) == 7
    assert pro(params(conv_k=None)) == 1
    assert pro(params(rope_base=-1.0)) == 6
    assert pro(params(rope_base=float("nan"))) == 6
    assert pro(params(pos0=-3)) == 6
    assert pro(params(pos0=2**31 - 69)) == 6       # the last position past 2^31 - 1
    assert pro(params(norm_bias=None)) == 1
    assert pro(params(norm_eps=-1.0)) == 6
    assert pro(params(conv_q=addr(20, 4).value)) == 4
    assert pro(q=None) == 1
    assert pro(fq=1) == 5                          # an output over an input
    assert pro(fk=5) == 5                          # two outputs over each other
    assert pro(st_in=addr(30), st_out=addr(30)) == 5   # the two states in one buffer
    assert pro(st_out=addr(1)) == 5                # the new state over k
    assert pro(d=desc(Dv=32, N=0)) == 2
    g = lambda o, gt, out: ia.lib.ia_block_gate(ctypes.byref(d), o, gt, out, None)
    assert g(addr(0), None, addr(2)) == 1
    assert g(addr(0), addr(1), addr(1)) == 5      # out over the gate
    assert g(addr(0), addr(1), addr(0, 64)) == 5  # out over part of o
    assert g(addr(0, 8), addr(1), addr(2)) == 4


def test_block_decode_step_validation():
    d = desc(Dv=32)   # B=2, H=3, F=32, Dv=32, M=16
    W = 4

    def params(**kw):
        p = dict(conv_width=W, conv_q=addr(20).value, conv_k=addr(21).value,
                 conv_v=addr(22).value, rope_base=1e4, pos0=9, norm_gain=addr(23).value,
                 norm_bias=addr(24).value, norm_eps=1e-6)
        p.update(kw)
        return ia.IABlockParams(**p)

    def step(p=None, d=d, q=0, st_in=None, st_out=None, gate=None, out=5, st=None):
        return ia.lib.ia_block_decode_step(
            ctypes.byref(d), None if p is False else ctypes.byref(p or params()),
            None if q is None else addr(q), addr(1), addr(2), st_in, st_out, gate,
            addr(3), addr(4), st or state(), addr(out), None)
    assert step(False) == 1
    assert step(q=None) == 1
    assert step(params(conv_width=9)) == 7
    assert step(params(conv_k=None)) == 1
    assert step(params(pos0=-1)) == 6
    assert step(params(norm_gain=None)) == 1
    assert step(params(norm_eps=float("inf"))) == 6
    assert step(params(norm_bias=addr(24, 4).value)) == 4
    assert step(gate=addr(30, 8)) == 4
    assert step(st_in=addr(31, 8)) == 4
    assert step(d=desc(Dv=32, bidir=True)) == 7
    assert step(d=desc(Dv=32, identity_features=True)) == 7
    assert step(out=1) == 5                          # the output over k
    assert step(gate=addr(5)) == 5                   # the output over the gate
    assert step(st_in=addr(30), st_out=addr(30)) == 5   # the two convolution states in one
    assert step(st_out=addr(5)) == 5                 # the new convolution state over the output
    assert step(st_out=addr(23)) == 5                # ... over the normalisation gain


def test_gated_variants_validation():
    d = desc(Dv=32)
    g = lambda *a: ia.lib.ia_prefill_fwd_gated(ctypes.byref(d), *a)
    base = [addr(0), addr(1), addr(2), addr(20), addr(21), addr(3), addr(4), state(), addr(5),
            addr(6), 1 << 40, None]
    for i in (3, 4):                         # a gate array missing
        a = list(base)
        a[i] = P(0)
        assert g(*a) == 1
    a = list(base)
    a[3] = addr(20, 8)                       # misaligned gate array
    assert g(*a) == 4
    a = list(base)
    a[8] = addr(20, 64)                      # o overlapping the write gates
    assert g(*a) == 5
    assert ia.lib.ia_decode_step_gated(ctypes.byref(d), addr(0), addr(1), addr(2), P(0),
                                       addr(21), addr(3), addr(4), state(), addr(5), None) == 1
    assert ia.lib.ia_decode_step_gated(ctypes.byref(d), addr(0), addr(1), addr(2), addr(20),
                                       addr(21), addr(3), addr(4), state(), addr(21, 16),
                                       None) == 5
    # workspace: fp32 inputs, the token-sequential path's (one state, rounded up to 256 bytes);
    # bf16 inputs on a chunk shape, the chunked plan's (the plain prefill's, when no device
    # reports the kernels' occupancy)
    B, H, M, F, D = 2, 3, 16, 32, 32
    want = (B * H * M * (F + D + 1) * 8 + 255) // 256 * 256
    d32 = desc(Dv=32, in_dtype=ia.IA_F32)
    assert ia.lib.ia_prefill_gated_workspace_bytes(ctypes.byref(d32)) == want
    if not _has_device():
        assert (ia.lib.ia_prefill_gated_workspace_bytes(ctypes.byref(d)) ==
                ia.lib.ia_prefill_workspace_bytes(ctypes.byref(d)))
