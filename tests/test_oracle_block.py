"""Pins of the block-edge oracle (oracle/block.py) against closed forms, invariants and
hand-computed values, and planted mistakes that each fail one of them (CPU only)."""
import math
import types

import numpy as np
import pytest

import oracle.block as blk


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- SiLU

def test_silu_values_and_odd_part():
    # SiLU(0) = 0, SiLU(x) - SiLU(-x) = x (sigmoid(x) + sigmoid(-x) = 1), SiLU(x) -> x for
    # large x, and one value by hand: SiLU(1) = 1 / (1 + e^-1).
    x = _rng(1).standard_normal(50) * 4
    assert blk.silu(0.0) == 0.0
    np.testing.assert_allclose(blk.silu(x) - blk.silu(-x), x, rtol=0, atol=1e-12)
    assert abs(blk.silu(40.0) - 40.0) < 1e-12
    assert abs(blk.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


# ---------------------------------------------------------------- short convolution

def test_conv_delta_tap_shifts_with_state():
    # A single tap at lag tau returns the sequence tau tokens back, the state supplying the
    # tokens before the first; the new state is the last W-1 tokens.
    N, C, W = 9, 3, 4
    x = _rng(2).standard_normal((N, C))
    st = _rng(3).standard_normal((W - 1, C))
    full = np.concatenate([st, x])
    for tau in range(W):
        w = np.zeros((C, W))
        w[:, tau] = 1.0
        y, ns = blk.short_conv(x, w, st)
        np.testing.assert_array_equal(y, full[W - 1 - tau:W - 1 - tau + N])
        np.testing.assert_array_equal(ns, full[-(W - 1):])


def test_conv_is_bilinear_and_split_invariant():
    N, C, W = 12, 4, 3
    r = _rng(4)
    x1, x2 = r.standard_normal((N, C)), r.standard_normal((N, C))
    w1, w2 = r.standard_normal((C, W)), r.standard_normal((C, W))
    y = lambda x, w: blk.short_conv(x, w)[0]
    np.testing.assert_allclose(y(2 * x1 - x2, w1), 2 * y(x1, w1) - y(x2, w1), atol=1e-12)
    np.testing.assert_allclose(y(x1, w1 + w2), y(x1, w1) + y(x1, w2), atol=1e-12)
    # two calls carrying the state equal one call
    a, s = blk.short_conv(x1[:5], w1)
    b, _ = blk.short_conv(x1[5:], w1, s)
    np.testing.assert_allclose(np.concatenate([a, b]), y(x1, w1), atol=1e-12)


# ---------------------------------------------------------------- RoPE

def test_rope_hand_values_and_position_zero():
    # F = 4, base 100: pair 0 turns by p rad, pair 1 by p / 10 rad.
    x = np.array([[1.0, 0.0, 0.0, 2.0]])
    out = blk.rope(x, [3.0], 100.0)
    np.testing.assert_allclose(out[0], [math.cos(3), math.sin(3), -2 * math.sin(0.3),
                                        2 * math.cos(0.3)], atol=1e-15)
    y = _rng(5).standard_normal((4, 8))
    np.testing.assert_array_equal(blk.rope(y, [0] * 4, 1e4), y)


def test_rope_keeps_pair_norms_and_depends_on_offsets_only():
    r = _rng(6)
    q, k = r.standard_normal((1, 16)), r.standard_normal((1, 16))
    rq = blk.rope(q, [7.0], 1e4)
    np.testing.assert_allclose((rq ** 2).reshape(8, 2).sum(1), (q ** 2).reshape(8, 2).sum(1),
                               rtol=1e-13)
    dot = lambda m, n: float((blk.rope(q, [m], 1e4) @ blk.rope(k, [n], 1e4).T)[0, 0])
    assert abs(dot(11, 4) - dot(107, 100)) < 1e-11
    assert abs(dot(11, 4) - float((blk.rope(q, [7], 1e4) @ k.T)[0, 0])) < 1e-11


# ---------------------------------------------------------------- RMSNorm with bias

def test_rmsnorm_unit_rms_scale_invariance_and_bias():
    r = _rng(7)
    z = r.standard_normal((5, 12)) * 3
    one, zero = np.ones(12), np.zeros(12)
    out = blk.rmsnorm_bias(z, one, zero, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(blk.rmsnorm_bias(4.5 * z, one, zero, 0.0), out, rtol=1e-13)
    g, b = r.standard_normal(12), r.standard_normal(12)
    np.testing.assert_allclose(blk.rmsnorm_bias(z, g, b, 0.0), g * out + b, rtol=1e-13)
    # hand case: z = [3, 4] has rms sqrt(12.5)
    np.testing.assert_allclose(blk.rmsnorm_bias(np.array([[3.0, 4.0]]), [1, 1], [0, 0], 0.0),
                               [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)


# ---------------------------------------------------------------- the prologue and the gate

def test_prologue_plain_is_the_feature_map():
    # no convolution, no RoPE, no norm: phi(q), phi(k) and v unchanged
    r = _rng(8)
    q, k, v = r.standard_normal((2, 5, 3, 4)), r.standard_normal((2, 5, 3, 4)), r.standard_normal((2, 5, 3, 6))
    fq, fk, vo, st = blk.prologue(q, k, v)
    np.testing.assert_array_equal(fq, blk.feature(q))
    np.testing.assert_array_equal(fk, blk.feature(k))
    np.testing.assert_array_equal(vo, v)
    assert st is None


def _params(H, F, D, W, seed):
    r = _rng(seed)
    conv = (r.standard_normal((H, F, W)) * 0.5, r.standard_normal((H, F, W)) * 0.5,
            r.standard_normal((H, D, W)) * 0.5)
    norm = (1.0 + 0.1 * r.standard_normal((H, F + D)), 0.1 * r.standard_normal((H, F + D)))
    return conv, norm


def test_prologue_stages_compose_and_split():
    B, N, H, F, D, W = 1, 10, 2, 4, 6, 3
    r = _rng(9)
    q, k, v = r.standard_normal((B, N, H, F)), r.standard_normal((B, N, H, F)), r.standard_normal((B, N, H, D))
    conv, norm = _params(H, F, D, W, 10)
    fq, fk, vo, st = blk.prologue(q, k, v, conv, None, 1e4, 5, norm, 1e-6)
    # by hand from the stages, head 1
    h = 1
    raw = np.concatenate([q[0, :, h], k[0, :, h], v[0, :, h]], axis=1)
    w = np.concatenate([conv[0][h], conv[1][h], conv[2][h]])
    y = blk.silu(blk.short_conv(raw, w)[0])
    pos = 5 + np.arange(N)
    eq = blk.feature(blk.rope(y[:, :F], pos, 1e4))
    ek = blk.feature(blk.rope(y[:, F:2 * F], pos, 1e4))
    z = blk.rmsnorm_bias(np.concatenate([ek, y[:, 2 * F:]], 1), norm[0][h], norm[1][h], 1e-6)
    np.testing.assert_allclose(fq[0, :, h], eq, rtol=1e-14)
    np.testing.assert_allclose(fk[0, :, h], z[:, :F], rtol=1e-14)
    np.testing.assert_allclose(vo[0, :, h], z[:, F:], rtol=1e-14)
    # two calls carrying the convolution state and the position equal one call
    a = blk.prologue(q[:, :4], k[:, :4], v[:, :4], conv, None, 1e4, 5, norm, 1e-6)
    b = blk.prologue(q[:, 4:], k[:, 4:], v[:, 4:], conv, a[3], 1e4, 9, norm, 1e-6)
    for i in range(3):
        np.testing.assert_allclose(np.concatenate([a[i], b[i]], axis=1), (fq, fk, vo)[i],
                                   rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b[3], st, rtol=0)


def test_gate_values():
    o = _rng(11).standard_normal((3, 4))
    np.testing.assert_array_equal(blk.gate(o, np.zeros((3, 4))), np.zeros((3, 4)))
    np.testing.assert_allclose(blk.gate(o, np.full((3, 4), 60.0)), 60.0 * o, rtol=1e-12)
    np.testing.assert_allclose(blk.gate(o, np.ones((3, 4))), o / (1 + math.exp(-1)), rtol=1e-15)


# ---------------------------------------------------------------- planted mistakes

BLOCK_MUTANTS = {
    "silu_as_sigmoid": ("return x / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(-x))"),
    "conv_anticausal": ("y[n] += w[:, tau] * full[n + W - 1 - tau]",
                        "y[n] += w[:, tau] * full[min(n + W - 1 + tau, len(full) - 1)]"),
    "rope_half_pairs": ("a, b = x[n, 2 * i], x[n, 2 * i + 1]", "a, b = x[n, i], x[n, i + F // 2]"),
    "rope_sign": ("out[n, 2 * i] = a * c - b * s", "out[n, 2 * i] = a * c + b * s"),
    "rms_without_mean": ("r = np.sqrt(np.mean(z * z, axis=1, keepdims=True) + eps)",
                         "r = np.sqrt(np.sum(z * z, axis=1, keepdims=True) + eps)"),
    "bias_inside_scale": ("* z / r + np.asarray(b, dtype=np.float64)[None, :]",
                          "* (z + np.asarray(b, dtype=np.float64)[None, :]) / r"),
    "gate_on_sigmoid": ("return np.asarray(o, dtype=np.float64) * silu(g)",
                        "return np.asarray(o, dtype=np.float64) / (1.0 + np.exp(-np.asarray(g)))"),
    "state_newest_first": ("full[len(full) - (W - 1):].copy()", "full[len(full) - (W - 1):][::-1].copy()"),
}


@pytest.mark.parametrize("mutant", sorted(BLOCK_MUTANTS))
def test_planted_block_mistake_fails_a_pin(mutant):
    old, new = BLOCK_MUTANTS[mutant]
    src = open(blk.__file__).read()
    assert src.count(old) == 1, mutant
    mod = types.ModuleType("block_mutant")
    exec(compile(src.replace(old, new), "block_mutant", "exec"), mod.__dict__)
    pins = [test_silu_values_and_odd_part, test_conv_delta_tap_shifts_with_state,
            test_conv_is_bilinear_and_split_invariant, test_rope_hand_values_and_position_zero,
            test_rope_keeps_pair_norms_and_depends_on_offsets_only,
            test_rmsnorm_unit_rms_scale_invariance_and_bias, test_prologue_plain_is_the_feature_map,
            test_prologue_stages_compose_and_split, test_gate_values]
    failed = 0
    saved = blk.__dict__.copy()
    try:
        blk.__dict__.update({k: v for k, v in mod.__dict__.items() if callable(v)})
        for pin in pins:
            try:
                pin()
            except AssertionError:
                failed += 1
    finally:
        blk.__dict__.clear()
        blk.__dict__.update(saved)
    assert failed > 0, f"planted mistake {mutant} passed every pin"
