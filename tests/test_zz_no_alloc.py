"""ia_prefill_fwd_noalloc (no workspace argument, no allocation; its workspace is the library's
fixed device array) against ia_prefill_fwd on the same inputs, through the C ABI: two calls in
a row on the shared array, the second smaller, then a bidirectional call; and a call whose
workspace exceeds the array is refused without touching its outputs."""
import numpy as np
import pytest

import ia_workloads as W
import oracle
from helpers import dev, tag

pytestmark = pytest.mark.gpu


def _pair(ia, torch, B, H, N, F, M, seed, with_state, bidir=False, out=None):
    out = torch.float32 if out is None else out
    inp = W.make_inputs(B, H, N, F, F, M, dtype="bf16", seed=seed)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in "qkv")
    lam, beta = dev(inp["lam"]), dev(inp["beta"])
    desc = ia.make_desc(B, H, N, F, F, M, ia.IA_BF16, ia.dtype_code(out), bidir=bidir)
    assert ia.ia_prefill_workspace_bytes(desc) <= ia.NOALLOC_SCRATCH_BYTES
    st_a = st_b = None
    if with_state:
        pre = W.make_inputs(B, H, 12, F, F, M, dtype="bf16", seed=seed + 1)
        st0 = oracle.prefill(pre["q"], pre["k"], pre["v"], inp["lam"], inp["beta"],
                             threads=8)[3]
        st_a = tuple(dev(x) for x in st0)
        st_b = tuple(dev(x) for x in st0)
    o_a = torch.full((B, N, H, F), 7.0, dtype=out, device="cuda")
    o_b = torch.full((B, N, H, F), -7.0, dtype=out, device="cuda")
    ws = torch.empty(max(ia.ia_prefill_workspace_bytes(desc), 16), dtype=torch.uint8,
                     device="cuda")
    tag(f"noalloc vs prefill B={B} H={H} N={N} F={F} M={M} state={with_state} bidir={bidir}")
    ia.ia_prefill_fwd(desc, q, k, v, lam, beta, st_a, o_a, ws)
    ia.ia_prefill_fwd_noalloc(desc, q, k, v, lam, beta, st_b, o_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    if with_state:
        assert all(torch.equal(x, y) for x, y in zip(st_a, st_b))


def test_noalloc_equals_prefill_two_calls_then_smaller():
    import torch
    import ssm_sequence_mixer_amd as ia
    # the 1.3B-shaped layer with a state (four segments, the state copy, 21 MiB of workspace)
    _pair(ia, torch, 4, 16, 2048, 128, 64, seed=801, with_state=True, out=torch.bfloat16)
    # then a smaller call on the same array: many segments through the carry kernel
    _pair(ia, torch, 1, 2, 300, 64, 32, seed=802, with_state=True)
    # and a bidirectional one, no state
    _pair(ia, torch, 2, 3, 333, 32, 32, seed=803, with_state=False, bidir=True)


def test_noalloc_refuses_a_workspace_beyond_its_array():
    import torch
    import ssm_sequence_mixer_amd as ia
    B, H, N, F, M = 64, 16, 32, 128, 64        # the decode workload's prefix at B=64
    desc = ia.make_desc(B, H, N, F, F, M, ia.IA_BF16, ia.IA_F32)
    assert ia.ia_prefill_workspace_bytes(desc) > ia.NOALLOC_SCRATCH_BYTES
    z = torch.zeros((B, N, H, F), dtype=torch.bfloat16, device="cuda")
    lam = dev(W.s4d_lin(np.full(H, 0.01), M))
    beta = dev(np.ones((H, M), np.complex64))
    o = torch.full((B, N, H, F), 3.0, dtype=torch.float32, device="cuda")
    tag("noalloc oversize call")
    with pytest.raises(ia.IAError) as e:
        ia.ia_prefill_fwd_noalloc(desc, z, z, z, lam, beta, None, o)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
