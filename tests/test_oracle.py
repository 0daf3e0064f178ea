"""Pins of the CPU oracle to facts other than itself (no GPU).

Each pin is a property fixed by the pages' definition of the layer or by mathematics, not a
retyping of the oracle's formula:
  hand    values worked by hand (tests/golden/hand_cases.json)
  P1      the recurrence equals the unrolled double sum over s <= t and modes (oracle/brute.py)
  P3      a scan equals the same tokens fed one decode step at a time, from any split point
  P4      eta_t has the closed form beta (1 - lambda^(t+1)) / (1 - lambda)  (beta (t+1) at 1)
  P5      with lambda_m the M-th roots of unity, beta = 1 and 2t < M, o_t = v_t exactly
          (the mode sum is a DFT that keeps only s = s' = t); a conjugated readout would
          give causal linear attention instead
  P6      one real mode: o_t is the exponential moving average of v, independent of q and k
  P7      o is linear in v; invariant under a common real scaling of beta
  P8      the bidirectional layer commutes with reversing the sequence
  P9      forced clamp: beta = i with real lambda makes Re(den) < 0, so o = num / clamp
  P10     the state holds 2(F+Dv)M + 2M reals per (b,h)  (summary page §D.2 plus eta)
The mutant test at the end builds deliberately broken copies of ia_oracle.c and checks that
each one fails at least one pin.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _rand_case(rng, N, F, D, M, complex_beta=True, rmin=0.6):
    q = rng.standard_normal((N, F))
    k = rng.standard_normal((N, F))
    v = rng.standard_normal((N, D))
    r = rng.uniform(rmin, 1.0, M)
    th = rng.uniform(-np.pi, np.pi, M)
    lam = r * np.exp(1j * th)
    beta = (rng.standard_normal(M) + 1j * rng.standard_normal(M)) if complex_beta else np.ones(M)
    return q, k, v, lam, beta


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- pin functions
# Each takes a scan callable (the oracle, or a broken copy) and returns the error it sees.

def pin_hand(scan):
    worst = 0.0
    for c in json.load(open(GOLD))["cases"]:
        lam = np.array([complex(*x) for x in c["lam"]])
        beta = np.array([complex(*x) for x in c["beta"]])
        o, num, den, (U, G, e) = scan(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                      lam, beta, None, c["clamp"])
        cpl = lambda a: np.array(a)[..., 0] + 1j * np.array(a)[..., 1]
        for got, want in ((o, c["o"]), (num, c["num"]), (den, c["den"]), (U, cpl(c["U_final"])),
                          (G, cpl(c["G_final"])), (e, cpl(c["e_final"]))):
            worst = max(worst, _rel(got, want))
    return worst


def pin_brute(scan, seed=0):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (N, F, D, M) in ((23, 3, 5, 4), (9, 1, 2, 3), (31, 4, 4, 2)):
        q, k, v, lam, beta = _rand_case(rng, N, F, D, M)
        o, num, den, _ = scan(q, k, v, lam, beta, None, 1e-6)
        ob, nb, db = brute.layer(q, k, v, lam, beta, 1e-6)
        worst = max(worst, _rel(num, nb), _rel(den, db), _rel(o, ob))
    return worst


def pin_eta_closed_form(scan, seed=1):
    rng = np.random.default_rng(seed)
    N, F, D, M = 40, 2, 2, 6
    q, k, v, lam, beta = _rand_case(rng, N, F, D, M)
    lam[0] = 1.0  # the lambda = 1 branch
    _, _, _, (_, _, e) = scan(q, k, v, lam, beta, None, 1e-6)
    want = np.where(np.abs(lam - 1) > 0, beta * (1 - lam ** N) / np.where(lam == 1, 1, 1 - lam),
                    beta * N)
    return _rel(e, want)


def pin_dft_roots(scan, seed=2):
    rng = np.random.default_rng(seed)
    M, N, F, D = 64, 32, 5, 7   # 2t <= 62 < M
    q, k, v, _, _ = _rand_case(rng, N, F, D, M)
    lam = np.exp(2j * np.pi * np.arange(M) / M)
    o, _, _, _ = scan(q, k, v, lam, np.ones(M), None, 1e-6)
    return _rel(o, v)


def pin_ema(scan, seed=3):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for lam0 in (0.9, 1.0):
        q, k, v, _, _ = _rand_case(rng, 50, 3, 4, 1)
        o, _, _, _ = scan(q, k, v, np.array([lam0]), np.ones(1), None, 1e-6)
        w = np.array([[lam0 ** (t - s) if s <= t else 0.0 for s in range(50)] for t in range(50)])
        want = (w @ v) / w.sum(1, keepdims=True)
        worst = max(worst, _rel(o, want))
    return worst


def pin_clamp(scan, seed=4):
    rng = np.random.default_rng(seed)
    N, F, D, M = 12, 3, 3, 4
    q, k, v, _, _ = _rand_case(rng, N, F, D, M)
    lam = rng.uniform(0.5, 0.99, M).astype(complex)
    beta = 1j * np.ones(M)
    o, num, den, _ = scan(q, k, v, lam, beta, None, 1e-6)
    if not np.all(den < 0):
        return np.inf
    return _rel(o, num / 1e-6)


PINS = {"hand": pin_hand, "brute": pin_brute, "eta": pin_eta_closed_form,
        "dft": pin_dft_roots, "ema": pin_ema, "clamp": pin_clamp}
TOL = 1e-9


# ---------------------------------------------------------------- the pins on the oracle

@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    err = PINS[name](oracle.scan)
    assert err < TOL, f"{name}: {err}"


def test_brute_dft_conjugate_reading_is_linear_attention():
    # The conjugate-transpose reading of Fq U^T would turn the DFT case into causal linear
    # attention; check that brute force (independent of the oracle) tells the two apart.
    rng = np.random.default_rng(5)
    M, N, F, D = 64, 20, 4, 3
    q, k, v, _, _ = _rand_case(rng, N, F, D, M)
    lam = np.exp(2j * np.pi * np.arange(M) / M)
    o, _, _ = brute.layer(q, k, v, lam, np.ones(M))
    assert _rel(o, v) < 1e-12
    S = brute.feature(q) @ brute.feature(k).T
    S = np.tril(S)
    lin = (S @ v) / S.sum(1, keepdims=True)
    assert _rel(o, lin) > 1e-2


def test_scan_equals_decode_steps_and_resume():
    rng = np.random.default_rng(6)
    B, N, H, F, D, M = 2, 17, 3, 4, 5, 6
    q = rng.standard_normal((B, N, H, F))
    k = rng.standard_normal((B, N, H, F))
    v = rng.standard_normal((B, N, H, D))
    lam = rng.uniform(0.7, 1, (H, M)) * np.exp(1j * rng.uniform(-3, 3, (H, M)))
    beta = rng.standard_normal((H, M)) + 1j * rng.standard_normal((H, M))
    o_full, _, _, st_full = oracle.prefill(q, k, v, lam, beta)
    for split in (0, 1, 9, 16):
        o_a, _, _, st = oracle.prefill(q[:, :split], k[:, :split], v[:, :split], lam, beta) \
            if split else (np.zeros((B, 0, H, D)), None, None, None)
        outs = [o_a]
        for t in range(split, N):
            if st is None:
                st = tuple(np.zeros(s, np.complex128) for s in ((B, H, M, F), (B, H, M, D), (B, H, M)))
            ot, st = oracle.decode_step(q[:, t], k[:, t], v[:, t], lam, beta, st)
            outs.append(ot[:, None])
        o = np.concatenate(outs, axis=1)
        assert _rel(o, o_full) < 1e-12
        for a, b in zip(st, st_full):
            assert _rel(a, b) < 1e-12


def test_linear_in_v_and_beta_scale_invariance():
    rng = np.random.default_rng(7)
    N, F, D, M = 30, 4, 3, 5
    q, k, v1, _, beta = _rand_case(rng, N, F, D, M, complex_beta=False)
    # S4D-Lin-shaped modes keep Re(den) well above the clamp, where the invariance is exact
    lam = np.exp(0.05 * (-0.5 + 1j * np.pi * np.arange(M)))
    v2 = rng.standard_normal((N, D))
    o1, _, den1, _ = oracle.scan(q, k, v1, lam, beta)
    assert np.all(den1 > 1e-3)
    o2 = oracle.scan(q, k, v2, lam, beta)[0]
    o12 = oracle.scan(q, k, 2.5 * v1 - 0.75 * v2, lam, beta)[0]
    assert _rel(o12, 2.5 * o1 - 0.75 * o2) < 1e-11
    o_scaled = oracle.scan(q, k, v1, lam, 3.0 * beta)[0]
    assert _rel(o_scaled, o1) < 1e-12


def test_bidir_flip_symmetry():
    rng = np.random.default_rng(8)
    B, N, H, F, D, M = 1, 21, 2, 3, 4, 5
    q = rng.standard_normal((B, N, H, F))
    k = rng.standard_normal((B, N, H, F))
    v = rng.standard_normal((B, N, H, D))
    lam = rng.uniform(0.7, 1, (H, M)) * np.exp(1j * rng.uniform(-3, 3, (H, M)))
    beta = np.ones((H, M), complex)
    fl = lambda a: np.ascontiguousarray(a[:, ::-1])
    o = oracle.bidir(q, k, v, lam, beta)
    o_fl = oracle.bidir(fl(q), fl(k), fl(v), lam, beta)
    assert _rel(o_fl, o[:, ::-1]) < 1e-12
    # and it is the sum of the two causal passes, each normalised on its own
    fwd = brute.layer_batched(q, k, v, lam, beta)
    rev = brute.layer_batched(fl(q), fl(k), fl(v), lam, beta)[:, ::-1]
    assert _rel(o, fwd + rev) < 1e-10


def test_state_size():
    B, N, H, F, D, M = 1, 3, 1, 6, 10, 4
    _, _, _, (U, G, e) = oracle.prefill(np.zeros((B, N, H, F)), np.zeros((B, N, H, F)),
                                        np.zeros((B, N, H, D)), np.ones((H, M), complex),
                                        np.ones((H, M), complex))
    reals = 2 * (U[0, 0].size + G[0, 0].size + e[0, 0].size)
    assert reals == 2 * (F + D) * M + 2 * M


def test_nan_propagates():
    q = np.zeros((3, 2)); k = np.zeros((3, 2)); v = np.ones((3, 2))
    k[1, 0] = np.nan
    o = oracle.scan(q, k, v, np.array([0.5, 0.9]), np.ones(2))[0]
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1:]))


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "conjugate_readout": ("a += feature(qt[r]) * uc;", "a += feature(qt[r]) * conj(uc);"),
    "exclusive_readout": ("a += feature(qt[r]) * uc;",
                          "a += feature(qt[r]) * (uc - bm * feature(kt[r]));"),
    "keys_from_queries": ("bm * feature(kt[r]);", "bm * feature(qt[r]);"),
    "value_beta_dropped": ("gc = l * gc + bm * vt[j];", "gc = l * gc + vt[j];"),
    "lambda_conjugated": ("double complex l = lam[2 * m] + I * lam[2 * m + 1];",
                          "double complex l = lam[2 * m] - I * lam[2 * m + 1];"),
    "den_modulus": ("double d = creal(denc);", "double d = cabs(denc);"),
    "no_clamp": ("double dc = d < clamp ? clamp : d;", "double dc = d;"),
    "elu_without_one": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x);"),
    "eta_not_decayed": ("ec = l * ec + bm;", "ec = ec + bm;"),
    "numerator_conj_a": ("numc[j] += a * gc;", "numc[j] += conj(a) * gc;"),
    "feature_index_shift": ("a += feature(qt[r]) * uc;",
                            "a += feature(qt[(r + 1) % F]) * uc;"),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(mutant, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    lib = oracle.load_library(str(so))
    scan = lambda *a: oracle.scan(*a, lib=lib)
    errs = {name: fn(scan) for name, fn in PINS.items()}
    assert any(not (e < TOL) for e in errs.values()), f"{mutant} passed every pin: {errs}"


# ---------------------------------------------------------------- readout matrix

def _rm_case(seed, N=9, F=3, D=4, M=5):
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal((N, F)), rng.standard_normal((N, F)), rng.standard_normal((N, D))
    lam = rng.uniform(0.5, 0.95, M) * np.exp(1j * rng.uniform(-1, 1, M))
    beta = 1.0 + 0.3j * rng.uniform(-1, 1, M)
    R = np.eye(M) + 0.3 * (rng.standard_normal((M, M)) + 1j * rng.standard_normal((M, M)))
    return q, k, v, lam, beta, R


def test_readout_matrix_identity_is_the_plain_layer():
    q, k, v, lam, beta, _ = _rm_case(21)
    o, num, den, st = oracle.scan_readout(q, k, v, lam, beta, np.eye(len(lam)))
    o2, num2, den2, st2 = oracle.scan(q, k, v, lam, beta)
    assert _rel(num, num2) < 1e-12 and _rel(den, den2) < 1e-12 and _rel(o, o2) < 1e-12
    assert max(_rel(a, b) for a, b in zip(st, st2)) < 1e-12


@pytest.mark.parametrize("seed", [22, 23])
def test_readout_matrix_matches_brute_force(seed):
    """The explicit double sum over s <= t, with (a R) in place of a (brute.layer)."""
    q, k, v, lam, beta, R = _rm_case(seed)
    o, num, den, _ = oracle.scan_readout(q, k, v, lam, beta, R)
    ob, nb, db = brute.layer(q, k, v, lam, beta, readout=R)
    assert _rel(num, nb) < 1e-10 and _rel(den, db) < 1e-10 and _rel(o, ob) < 1e-10


def test_readout_matrix_linearity():
    """num and den are real-linear in R (the state does not depend on it): R3 = 2 R1 - 0.5 R2
    gives 2 num1 - 0.5 num2, and likewise den."""
    q, k, v, lam, beta, R1 = _rm_case(24)
    R2 = _rm_case(25)[5]
    _, n1, d1, _ = oracle.scan_readout(q, k, v, lam, beta, R1)
    _, n2, d2, _ = oracle.scan_readout(q, k, v, lam, beta, R2)
    _, n3, d3, _ = oracle.scan_readout(q, k, v, lam, beta, 2.0 * R1 - 0.5 * R2)
    assert _rel(n3, 2.0 * n1 - 0.5 * n2) < 1e-10
    assert _rel(d3, 2.0 * d1 - 0.5 * d2) < 1e-10


READOUT_MUTANTS = {
    "readout_matrix_transposed": ("acc += av[m] * (R[((size_t)m * M + n) * 2] + I * R[((size_t)m * M + n) * 2 + 1]);",
                                  "acc += av[m] * (R[((size_t)n * M + m) * 2] + I * R[((size_t)n * M + m) * 2 + 1]);"),
    "readout_den_unmixed": ("for (int n = 0; n < M; ++n) dc += ar[n] * (e[2 * n] + I * e[2 * n + 1]);",
                            "for (int n = 0; n < M; ++n) dc += av[n] * (e[2 * n] + I * e[2 * n + 1]);"),
}


@pytest.mark.parametrize("mutant", sorted(READOUT_MUTANTS))
def test_planted_readout_mistake_fails_brute_force(mutant, tmp_path):
    src = open(oracle._SRC).read()
    old, new = READOUT_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    lib = oracle.load_library(str(so))
    q, k, v, lam, beta, R = _rm_case(22)
    o, num, den, _ = oracle.scan_readout(q, k, v, lam, beta, R, lib=lib)
    ob, nb, db = brute.layer(q, k, v, lam, beta, readout=R)
    assert not (_rel(num, nb) < 1e-10 and _rel(den, db) < 1e-10), f"{mutant} passed"


# ---------------------------------------------------------------- selective writing, memory decay
# ia_oracle_scan_gated: a write gate w_t on what token t writes (U, Gamma, eta) and a decay gate
# a_t scaling every mode's lambda at step t.  Pinned to the pinned plain layer (unit gates; a
# constant decay gate is the plain layer with a scaled lambda), to the explicit double sum with
# the gates' cumulative products (brute.layer(gates=...)), and to two invariances.

def _gate_case(seed, N=11, F=3, D=4, M=5):
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal((N, F)), rng.standard_normal((N, F)), rng.standard_normal((N, D))
    lam = rng.uniform(0.5, 0.95, M) * np.exp(1j * rng.uniform(-1, 1, M))
    beta = 1.0 + 0.3j * rng.uniform(-1, 1, M)
    w = rng.uniform(0.0, 1.5, N)
    a = rng.uniform(0.2, 1.0, N)
    return q, k, v, lam, beta, w, a


def test_gated_unit_gates_are_the_plain_layer():
    q, k, v, lam, beta, _, _ = _gate_case(31)
    ones = np.ones(len(q))
    o1, n1, d1, s1 = oracle.scan_gated(q, k, v, lam, beta, ones, ones)
    o2, n2, d2, s2 = oracle.scan(q, k, v, lam, beta)
    assert np.array_equal(n1, n2) and np.array_equal(d1, d2) and np.array_equal(o1, o2)
    assert all(np.array_equal(x, y) for x, y in zip(s1, s2))


@pytest.mark.parametrize("seed", [32, 33, 34])
def test_gated_matches_brute_force(seed):
    """The explicit double sum over s <= t with weight w_s prod_{s<u<=t} a_u lambda^(t-s),
    the products as exp of summed logs and lambda^n as exp(n Log lambda)."""
    q, k, v, lam, beta, w, a = _gate_case(seed)
    o, num, den, _ = oracle.scan_gated(q, k, v, lam, beta, w, a)
    ob, nb, db = brute.layer(q, k, v, lam, beta, gates=(w, a))
    assert _rel(num, nb) < 1e-10 and _rel(den, db) < 1e-10
    ok = db > 1e-6
    assert _rel(o[ok], ob[ok]) < 1e-10


def test_gated_constant_decay_is_a_scaled_lambda():
    """a_t = c at every step (w = 1) is the plain layer with modes c lambda."""
    q, k, v, lam, beta, _, _ = _gate_case(35)
    c = 0.83
    o1, n1, d1, s1 = oracle.scan_gated(q, k, v, lam, beta, np.ones(len(q)), np.full(len(q), c))
    o2, n2, d2, s2 = oracle.scan(q, k, v, c * lam, beta)
    assert _rel(n1, n2) < 1e-12 and _rel(d1, d2) < 1e-12
    assert max(_rel(x, y) for x, y in zip(s1, s2)) < 1e-12


def test_gated_zero_write_gate_drops_the_token():
    """w_t = 0: token t writes nothing, so its k_t and v_t change no output and no state."""
    q, k, v, lam, beta, w, a = _gate_case(36)
    t0 = 4
    w = w.copy()
    w[t0] = 0.0
    o1, _, _, s1 = oracle.scan_gated(q, k, v, lam, beta, w, a)
    k2, v2 = k.copy(), v.copy()
    k2[t0] += 3.0
    v2[t0] -= 5.0
    o2, _, _, s2 = oracle.scan_gated(q, k2, v2, lam, beta, w, a)
    assert _rel(o1, o2) < 1e-13 and max(_rel(x, y) for x, y in zip(s1, s2)) < 1e-13


def test_gated_common_write_scale():
    """Scaling every write gate by c scales U, Gamma, eta by c, so num and den by c^2 and o is
    unchanged wherever den stays above the clamp."""
    q, k, v, lam, beta, w, a = _gate_case(37)
    c = 1.7
    o1, n1, d1, _ = oracle.scan_gated(q, k, v, lam, beta, w, a)
    o2, n2, d2, _ = oracle.scan_gated(q, k, v, lam, beta, c * w, a)
    assert _rel(n2, c * c * n1) < 1e-12 and _rel(d2, c * c * d1) < 1e-12
    ok = (d1 > 1e-6) & (d2 > 1e-6)
    assert ok.any() and _rel(o1[ok], o2[ok]) < 1e-12


GATE_MUTANTS = {
    "decay_gate_on_the_write_too": ("const double complex wb = w * (beta[2 * m] + I * beta[2 * m + 1]);",
                                    "const double complex wb = at * w * (beta[2 * m] + I * beta[2 * m + 1]);"),
    "eta_not_gated": ("const double complex ec = l * (e[2 * m] + I * e[2 * m + 1]) + wb;",
                      "const double complex ec = l * (e[2 * m] + I * e[2 * m + 1]) + (beta[2 * m] + I * beta[2 * m + 1]);"),
    "value_write_not_gated": ("const double complex gc = l * (g[0] + I * g[1]) + wb * v[(size_t)t * D + j];",
                              "const double complex gc = l * (g[0] + I * g[1]) + (beta[2 * m] + I * beta[2 * m + 1]) * v[(size_t)t * D + j];"),
    "decay_gate_as_power": ("const double complex l = at * (lam[2 * m] + I * lam[2 * m + 1]);",
                            "const double complex l = cpow(lam[2 * m] + I * lam[2 * m + 1], at);"),
    "gates_one_token_late": ("const double w = wgate[t], at = dgate[t];",
                             "const double w = wgate[t > 0 ? t - 1 : 0], at = dgate[t > 0 ? t - 1 : 0];"),
}


@pytest.mark.parametrize("mutant", sorted(GATE_MUTANTS))
def test_planted_gate_mistake_fails_a_pin(mutant, tmp_path):
    src = open(oracle._SRC).read()
    old, new = GATE_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    lib = oracle.load_library(str(so))
    q, k, v, lam, beta, w, a = _gate_case(32)
    _, num, den, _ = oracle.scan_gated(q, k, v, lam, beta, w, a, lib=lib)
    _, nb, db = brute.layer(q, k, v, lam, beta, gates=(w, a))
    assert not (_rel(num, nb) < 1e-10 and _rel(den, db) < 1e-10), f"{mutant} passed"


# ---------------------------------------------------------------- denominator conditioning

def test_gated_condition_pins():
    """brute.gated_condition (the conditioning of the gated layer's readout sums, expanded over
    key pairs and modes): equal to an explicit loop over every (s, j, m) term on a tiny slice
    with signed gates, a zero decay and an initial state; exactly 1 when no term can be
    negative (real positive lambda, beta, gates and values); (1 + r^2) / |1 - r^2| for two equal
    real modes with beta = (1, i r), whose terms are those of the first mode times -r^2; never
    below the modes-only partial sum of den_condition.  (A term of a_m from the state is one
    entry U0[m, f] phi(q_t)[f]: the readout sums the entries like the keys.)"""
    r = np.random.default_rng(61)
    N, F, D, M = 7, 3, 2, 3
    q, k, v = (r.standard_normal((N, X)) for X in (F, F, D))
    lam = np.array([0.9 * np.exp(0.5j), 0.8 * np.exp(-2.0j), 0.97])
    beta = np.array([1.0, 0.4 - 0.9j, 1.5j])
    w = np.array([0.7, -0.4, 1.2, 0.0, 0.9, -1.1, 0.5])
    a = np.array([0.9, -0.6, 0.0, 0.8, -0.95, 0.7, 1.0])
    U0, G0, E0 = (r.standard_normal(sh) + 1j * r.standard_normal(sh) for sh in ((M, F), (M, D), (M,)))
    fq, fk = brute.feature(q), brute.feature(k)
    kd, kn = brute.gated_condition(q, k, v, lam, beta, w, a, state=(U0, G0, E0))
    for t in range(N):
        def g(s):   # w_s prod_{s<u<=t} a_u; s = -1: the state, carried by prod_{u<=t} a_u
            return (w[s] if s >= 0 else 1.0) * np.prod(a[s + 1: t + 1])
        den, dab = 0.0, 0.0
        num, nab = np.zeros(D), np.zeros(D)
        for m in range(M):
            # terms of a_m: one per key s, one per entry (m, f) of the state
            ta_all = [fq[t] @ fk[s] * g(s) * beta[m] * lam[m] ** (t - s) for s in range(t + 1)]
            ta_all += [fq[t][f] * U0[m, f] * g(-1) * lam[m] ** (t + 1) for f in range(F)]
            for ta in ta_all:
                for j in range(-1, t + 1):
                    if j >= 0:
                        te, tg = g(j) * beta[m] * lam[m] ** (t - j), g(j) * beta[m] * lam[m] ** (t - j) * v[j]
                    else:
                        te, tg = g(-1) * lam[m] ** (t + 1) * E0[m], g(-1) * lam[m] ** (t + 1) * G0[m]
                    den += np.real(ta * te)
                    dab += abs(ta) * abs(te)
                    num += np.real(ta * tg)
                    nab += abs(ta) * np.abs(tg)
        assert abs(kd[t] - dab / abs(den)) <= 1e-10 * kd[t], (t, kd[t], dab / abs(den))
        want_n = nab.max() / np.abs(num).max()
        assert abs(kn[t] - want_n) <= 1e-10 * want_n, (t, kn[t], want_n)
    # no cancellation possible: kappa = 1
    N = 30
    q, k = r.standard_normal((N, 6)), r.standard_normal((N, 6))
    vp = np.abs(r.standard_normal((N, 4)))
    wp, ap = r.uniform(0.1, 1.5, N), r.uniform(0.3, 1.0, N)
    kd, kn = brute.gated_condition(q, k, vp, np.array([0.9, 0.5, 0.99]), np.array([1.0, 0.3, 2.0]), wp, ap)
    assert np.all(np.abs(kd - 1.0) < 1e-12) and np.all(np.abs(kn - 1.0) < 1e-12)
    for rr in (0.5, 0.99, 1.01, 3.0):
        kd, kn = brute.gated_condition(q, k, vp, np.array([0.93, 0.93]), np.array([1.0, 1j * rr]), wp, ap)
        want = (1 + rr ** 2) / abs(1 - rr ** 2)
        assert np.all(np.abs(kd - want) <= 1e-9 * want) and np.all(np.abs(kn - want) <= 1e-9 * want)
    lam3 = np.array([0.95 * np.exp(0.3j), 0.9 * np.exp(-1.1j), 0.99])
    beta3 = np.array([1.0, 0.5 - 0.7j, 2.0j])
    kd, _ = brute.gated_condition(q, k, vp, lam3, beta3, wp, ap)
    for t in (0, 9, N - 1):
        assert kd[t] >= brute.den_condition(q, k, lam3, beta3, t, gates=(wp, ap))[0] * (1 - 1e-12)


def test_den_condition_pins():
    """brute.den_condition: its denominator is the layer's (with and without gates); kappa = 1
    when no term can cancel (real positive lambda and beta: every a_m eta_m > 0, the features
    being positive); and two equal modes with beta = (1, i r) give a_1 eta_1 = -r^2 a_0 eta_0,
    so kappa = (1 + r^2) / |1 - r^2| whatever the data."""
    r = np.random.default_rng(60)
    N, F, D = 40, 8, 4
    q, k, v = (r.standard_normal((N, X)) for X in (F, F, D))
    lam = np.array([0.95 * np.exp(0.3j), 0.9 * np.exp(-1.1j), 0.99])
    beta = np.array([1.0, 0.5 - 0.7j, 2.0j])
    gates = (r.uniform(0.2, 1.4, N), r.uniform(0.6, 1.0, N))
    for g in (None, gates):
        _, _, den = brute.layer(q, k, v, lam, beta, gates=g)
        for t in (0, 7, N - 1):
            kappa, d = brute.den_condition(q, k, lam, beta, t, gates=g)
            assert abs(d - den[t]) <= 1e-12 * max(1.0, abs(den[t]))
            assert kappa >= 1.0 - 1e-12
    lam_pos, beta_pos = np.array([0.9, 0.5, 0.99]), np.array([1.0, 0.3, 2.0])
    for t in (0, 11, N - 1):
        assert abs(brute.den_condition(q, k, lam_pos, beta_pos, t)[0] - 1.0) < 1e-12
    for rr in (0.5, 0.99, 1.01, 3.0):
        lam2 = np.array([0.93 * np.exp(0.4j)] * 2)
        beta2 = np.array([1.0, 1j * rr])
        for t in (3, N - 1):
            kappa = brute.den_condition(q, k, lam2, beta2, t)[0]
            want = (1 + rr ** 2) / abs(1 - rr ** 2)
            assert abs(kappa - want) <= 1e-9 * want, (rr, t, kappa, want)
