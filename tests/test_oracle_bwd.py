"""Pins of the oracle's backward pass (``oracle.scan_bwd``), CPU only.

The backward is pinned to the forward oracle, which the pins of ``test_oracle.py`` tie to the
pages, through central finite differences of a scalar loss L = sum(dO * o) (or
sum(dO * num) without the denominator) in fp64: every gradient entry (q, k, v, the real and
imaginary parts of lambda and beta, and the initial state) is compared with
(L(x + h) - L(x - h)) / 2h.  Cases: the smooth region (den well above the clamp), the clamped
region (den below the clamp everywhere, so o = num / clamp), and the readout without a
denominator.  Planted mistakes in a copy of the C source (a conjugate dropped, a term dropped,
an index shifted) must each fail one of these pins.
"""
import subprocess

import numpy as np
import pytest

import oracle

FD_TOL = 1e-6


def _case(seed, N=6, F=3, D=2, M=3, clamped=False):
    rng = np.random.default_rng(seed)

    def away_from_zero(shape):
        x = rng.standard_normal(shape)
        return np.where(np.abs(x) < 0.05, 0.05 * np.sign(x) + 0.05 * (x == 0), x)

    q, k = away_from_zero((N, F)), away_from_zero((N, F))
    v = rng.standard_normal((N, D))
    if clamped:
        # real lambda and beta = i: every term of Re den is -|.|^2 or 0, far below the clamp
        lam = rng.uniform(0.6, 0.95, M).astype(np.complex128)
        beta = np.full(M, 1j)
        st = None
    else:
        lam = rng.uniform(0.6, 0.95, M) * np.exp(1j * rng.uniform(-0.3, 0.3, M))
        beta = 1.0 + 0.2j * rng.uniform(-1, 1, M)
        st = (0.3 * (rng.uniform(0.5, 1, (M, F)) + 0.1j * rng.standard_normal((M, F))),
              0.3 * (rng.standard_normal((M, D)) + 1j * rng.standard_normal((M, D))),
              0.3 * (rng.uniform(0.5, 1, M) + 0.1j * rng.standard_normal(M)))
    dO = rng.standard_normal((N, D))
    return dict(q=q, k=k, v=v, lam=lam, beta=beta, st=st, dO=dO)


def _loss(c, no_den, clamp, scan=oracle.scan):
    o, num, den, _ = scan(c["q"], c["k"], c["v"], c["lam"], c["beta"], c["st"], clamp)
    return float(np.sum(c["dO"] * (num if no_den else o))), den


def _fd_errors(c, no_den=False, clamp=1e-6, bwd=oracle.scan_bwd):
    """max |analytic - finite difference| / max |analytic| for each gradient."""
    dq, dk, dv, dl, db, (dU, dG, de) = bwd(c["q"], c["k"], c["v"], c["lam"], c["beta"], c["dO"],
                                          c["st"], clamp, no_den)
    out = {}

    def fd_real(name, arr, grad, setter):
        fd = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            x0 = arr[idx]
            h = 1e-6 * max(1.0, abs(x0))
            vals = []
            for s in (1, -1):
                a = arr.copy()
                a[idx] = x0 + s * h
                vals.append(_loss(setter(a), no_den, clamp)[0])
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        out[name] = float(np.max(np.abs(fd - grad)) / max(np.max(np.abs(grad)), 1e-300))

    def with_key(key):
        return lambda a: {**c, key: a}

    fd_real("dq", c["q"], dq, with_key("q"))
    fd_real("dk", c["k"], dk, with_key("k"))
    fd_real("dv", c["v"], dv, with_key("v"))
    for key, g in (("lam", dl), ("beta", db)):
        z = c[key]
        fd_real(f"d{key}.re", z.real.copy(), g.real, lambda a, z=z, key=key: {**c, key: a + 1j * z.imag})
        fd_real(f"d{key}.im", z.imag.copy(), g.imag, lambda a, z=z, key=key: {**c, key: z.real + 1j * a})
    if c["st"] is not None:
        for i, (name, g) in enumerate((("dU0", dU), ("dG0", dG), ("de0", de))):
            z = c["st"][i]

            def put(a, i=i):
                st = list(c["st"])
                st[i] = a
                return {**c, "st": tuple(st)}

            fd_real(name + ".re", z.real.copy(), g.real, lambda a, z=z, put=put: put(a + 1j * z.imag))
            fd_real(name + ".im", z.imag.copy(), g.imag, lambda a, z=z, put=put: put(z.real + 1j * a))
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_backward_matches_finite_differences(seed):
    c = _case(seed)
    den = _loss(c, False, 1e-6)[1]
    assert den.min() > 0.05, "the case must stay in the smooth region of the clamp"
    errs = _fd_errors(c)
    assert max(errs.values()) < FD_TOL, errs


def test_backward_clamped_region_matches_finite_differences():
    c = _case(4, clamped=True)
    den = _loss(c, False, 1e-6)[1]
    assert den.max() < -1e-3, "every den must sit below the clamp"
    errs = _fd_errors(c)
    assert max(errs.values()) < FD_TOL, errs


@pytest.mark.parametrize("seed", [5, 6])
def test_backward_without_denominator_matches_finite_differences(seed):
    errs = _fd_errors(_case(seed), no_den=True)
    assert max(errs.values()) < FD_TOL, errs


def test_backward_longer_case_with_more_modes():
    errs = _fd_errors(_case(7, N=11, F=4, D=3, M=5))
    assert max(errs.values()) < FD_TOL, errs


BWD_MUTANTS = {
    "adjoint_not_conjugated": ("Ub[i] = conj(lm) * Ub[i];", "Ub[i] = lm * Ub[i];"),
    "den_term_dropped": ("double complex ga = dden * conj(et[m]);", "double complex ga = 0.0;"),
    "lambda_grad_wrong_state": ("gl += Ub[i] * conj(Up[i]);", "gl += Ub[i] * conj(Ut[i]);"),
    "key_grad_beta_unconjugated": ("dk[(size_t)t * F + r] += creal(Ub[i] * conj(bt));",
                                   "dk[(size_t)t * F + r] += creal(Ub[i] * bt);"),
    "feature_derivative_one": ("static double feature_grad(double x) { return x > 0.0 ? 1.0 : exp(x); }",
                               "static double feature_grad(double x) { return 1.0 + 0.0 * x; }"),
    "eta_adjoint_not_decayed": ("eb[m] = conj(lm) * eb[m];", "eb[m] = eb[m];"),
    "clamp_derivative_kept": ("dden = d >= clamp ? -gn / (c * c) : 0.0;",
                              "dden = -gn / (c * c);"),
    "beta_grad_value_dropped": ("gb += Gb[i] * v[(size_t)t * D + j];", "gb += 0.0 * Gb[i];"),
}


@pytest.mark.parametrize("mutant", sorted(BWD_MUTANTS))
def test_planted_backward_mistake_fails_a_pin(mutant, tmp_path):
    src = open(oracle._SRC).read()
    old, new = BWD_MUTANTS[mutant]
    assert src.count(old) == 1, f"mutation anchor for {mutant} not found once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(so),
                           str(path), "-lm"])
    lib = oracle.load_library(str(so))
    bwd = lambda *a: oracle.scan_bwd(*a, lib=lib)
    worst = 0.0
    for c, nd in ((_case(1), False), (_case(4, clamped=True), False), (_case(5), True)):
        worst = max(worst, max(_fd_errors(c, no_den=nd, bwd=bwd).values()))
    assert not worst < FD_TOL, f"{mutant} passed every finite-difference pin"


def test_bidirectional_backward_matches_finite_differences():
    """oracle.bidir_bwd against central differences of the bidirectional forward (oracle.bidir)
    on q, k, v and lambda."""
    rng = np.random.default_rng(9)
    B, N, H, F, D, M = 1, 6, 1, 3, 2, 3
    q, k = rng.standard_normal((B, N, H, F)), rng.standard_normal((B, N, H, F))
    v = rng.standard_normal((B, N, H, D))
    lam = (rng.uniform(0.6, 0.95, M) * np.exp(1j * rng.uniform(-0.3, 0.3, M)))[None]
    beta = (1.0 + 0.2j * rng.uniform(-1, 1, M))[None]
    dO = rng.standard_normal((B, N, H, D))
    loss = lambda q_, k_, v_, l_: float(np.sum(dO * oracle.bidir(q_, k_, v_, l_, beta)))
    dq, dk, dv, dl, _ = oracle.bidir_bwd(q, k, v, lam, beta, dO)
    errs = []
    for arr, grad, put in ((q, dq, lambda a: loss(a, k, v, lam)), (k, dk, lambda a: loss(q, a, v, lam)),
                           (v, dv, lambda a: loss(q, k, a, lam))):
        fd = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            h = 1e-6 * max(1.0, abs(arr[idx]))
            up, dn = arr.copy(), arr.copy()
            up[idx] += h
            dn[idx] -= h
            fd[idx] = (put(up) - put(dn)) / (2 * h)
        errs.append(np.max(np.abs(fd - grad)) / np.max(np.abs(grad)))
    fd = np.zeros(M, dtype=np.complex128)
    for m in range(M):
        for part, unit in ((0, 1.0), (1, 1j)):
            h = 1e-7
            up, dn = lam.copy(), lam.copy()
            up[0, m] += h * unit
            dn[0, m] -= h * unit
            d = (loss(q, k, v, up) - loss(q, k, v, dn)) / (2 * h)
            fd[m] += d if part == 0 else 1j * d
    errs.append(np.max(np.abs(fd - dl[0, 0])) / np.max(np.abs(dl[0, 0])))
    assert max(errs) < FD_TOL, errs
