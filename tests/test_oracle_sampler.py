"""Pins of the CPU reference's sampler, Philox generator and residual cascade.

LoopSpec page, section 2.2-2.3 (eq. 2-6 and the cascade): the committed token must be
distributed exactly as p_R; q = p_R gives certain acceptance; the residual mass equals
the total-variation distance; an open gate zeroes the residual at the first candidate;
double rejection is bounded by TV(p_d2, p_R) without the gate and by twice that with it.
"""

import os
import random
from fractions import Fraction

import numpy as np
import pytest

from oracle import decode, philox, sampler
from synth import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_philox_known_answers():
    rows = 0
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            assert philox.philox4x32_10(w[0:4], w[4:6]) == tuple(w[6:10])
            rows += 1
    assert rows == 3


def test_philox_uniform_keying():
    a = philox.uniform(2, 100, 0)
    assert a == philox.philox4x32_10((100, 0, 0, 0), (2, 0))[0]
    assert philox.uniform(2, 100, 1) != a and philox.uniform(3, 100, 0) != a
    assert philox.uniform((7 << 32) | 2, 100, 0) == philox.philox4x32_10((100, 0, 0, 0), (2, 7))[0]


def _fixed_rows(n, V, seed, **kw):
    return [sampler.fixed(p) for p in inputs.distributions(n, V, seed, **kw)]


def test_fixed_point_is_exact_floor():
    p = np.array([1.0, 0.5, 2.0 ** -40, 2.0 ** -41, 0.1, 0.0], np.float32)
    A = sampler.fixed(p)
    assert A[0] == 1 << 40 and A[1] == 1 << 39 and A[2] == 1 and A[3] == 0 and A[5] == 0
    assert A[4] == int(Fraction(float(np.float32(0.1))) * (1 << 40))


def test_sample_inverse_cdf_boundaries():
    A = [3, 0, 5, 2]                       # Z = 10
    W = 1 << 32
    for U, want in [(0, 0), (W * 3 // 10 - 1, 0), (-(-3 * W // 10), 2), (W - 1, 3)]:
        assert sampler.sample(A, U) == want
    # a zero-probability token is never drawn
    for U in range(0, W, W // 997):
        assert sampler.sample(A, U) != 1


def test_q_equals_p_always_accepts():
    for P in _fixed_rows(20, 50, 5, sparsity=0.3):
        for x in range(50):
            if P[x] == 0:
                continue
            for U in (0, 1 << 31, (1 << 32) - 1):
                assert sampler.accept(P, P, x, U)


def test_residual_mass_equals_tv():
    ps = inputs.distributions(30, 64, 11, sparsity=0.2)
    qs = inputs.distributions(30, 64, 12, sparsity=0.2)
    for p, q in zip(ps, qs):
        P, Q = sampler.fixed(p), sampler.fixed(q)
        tv = 0.5 * np.abs(p.astype(np.float64) - q.astype(np.float64)).sum()
        # sum [p - q]_+ = TV exactly when both sum to one; fp32 rows sum to 1 +- 64 ulp
        drift = abs(float(p.astype(np.float64).sum()) - 1) + abs(float(q.astype(np.float64).sum()) - 1)
        got = sum(sampler.resid(P, Q)) / float(1 << 40)
        assert abs(got - tv) <= drift + 64 * 2.0 ** -40


def test_non_residual_proposal_masks_the_first_candidate():
    """Table 3's non-residual second proposal: p_d2 renormalised without x~1, so x~2 != x~1;
    with the gate off it is drawn whenever p_d2 has mass outside x~1."""
    for seed in range(40):
        P1, P2 = _fixed_rows(2, 16, 300 + seed, peaked=2.0)
        x1 = sampler.draw1(P1, philox.uniform(seed, 3, 0))
        gate, x2 = sampler.draw2(P1, P2, x1, philox.uniform(seed, 3, 1), gated=False, residual=False)
        assert gate and x2 != x1 and P2[x2] > 0
    one_hot = [0] * 4
    one_hot[2] = 1 << 40
    assert sampler.draw2(one_hot, one_hot, 2, 12345, gated=False, residual=False) == (False, -1)


def test_gate_open_zeroes_residual_at_first_candidate():
    for seed in range(40):
        P1, P2 = _fixed_rows(2, 16, 100 + seed, peaked=2.0)
        x1 = sampler.draw1(P1, philox.uniform(seed, 3, 0))
        gate, x2 = sampler.draw2(P1, P2, x1, philox.uniform(seed, 3, 1))
        if gate:
            assert sampler.resid(P2, P1)[x1] == 0 and x2 != x1
        else:
            assert P2[x1] >= P1[x1] or sum(sampler.resid(P2, P1)) == 0


def _equal_total_rows(n, V, seed):
    """Integer distributions that each sum to exactly 2^40 (no fp32 rounding drift)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = []
    for _ in range(n):
        w = rng.exponential(size=V) * (rng.random(V) > 0.2)
        w[rng.integers(V)] += 0.5
        A = [int(x) for x in np.floor(w / w.sum() * (1 << 40))]
        A[int(np.argmax(w))] += (1 << 40) - sum(A)
        rows.append(A)
    return rows


MODES = {"single": (False, True, True), "gated": (True, True, True), "ungated": (True, False, True),
         "nonres-ungated": (True, False, False), "nonres-gated": (True, True, False)}


@pytest.mark.parametrize("mode", list(MODES))
def test_exact_commit_law_is_p_R(mode):
    """Exact law of the committed token (by counting uniform words) equals P_R/sum(P_R)
    (the method is lossless: section 2.2 and 2.3; Table 3's non-residual second proposal
    too).  With equal fixed-point totals the only error left is the 2^-32 granularity of
    the uniform words."""
    second, gated, residual = MODES[mode]
    rng = np.random.Generator(np.random.PCG64(7))
    for trial in range(12):
        V = int(rng.integers(2, 7))
        P_R, P_1, P_2 = _equal_total_rows(3, V, 1000 + trial)
        law = decode.exact_commit_distribution(P_R, P_1, P_2 if second else None, gated=gated, residual=residual)
        Z = sum(P_R)
        for v in range(V):
            assert abs(float(law[v]) - P_R[v] / Z) < 8 * V * 2.0 ** -32, (trial, v)
        assert sum(law) == 1


@pytest.mark.parametrize("mode", ["single", "gated"])
def test_exact_commit_law_fp32_inputs(mode):
    """With float32 readouts the fixed-point totals differ slightly (each row sums to one
    only up to float32 rounding); the law then deviates from P_R by at most the order of
    that mismatch."""
    for trial in range(12):
        V = 5
        P_R, P_1, P_2 = _fixed_rows(3, V, 1000 + trial, peaked=1.5, sparsity=0.2)
        law = decode.exact_commit_distribution(P_R, P_1, None if mode == "single" else P_2,
                                               gated=(mode == "gated"))
        Z = sum(P_R)
        mis = max(abs(sum(P_R) - sum(P_1)), abs(sum(P_R) - sum(P_2)), abs(sum(P_1) - sum(P_2))) / Z
        for v in range(V):
            assert abs(float(law[v]) - P_R[v] / Z) < 4 * mis + 8 * V * 2.0 ** -32, (trial, v)


def _double_reject_prob(P_R, P_1, P_2, gated):
    """Probability that both candidates are rejected (fall-back to the residual)."""
    W = 1 << 32

    def law_sample(A):
        Z = sum(A)
        out, c = [], 0
        for a in A:
            lo = -(-c * W // Z); c += a; hi = -(-c * W // Z)
            out.append(Fraction(min(hi, W) - min(lo, W), W))
        return out

    def acc(num, den):
        return Fraction(min(W, -(-num * W // den)), W) if den else Fraction(1)

    r1 = sampler.resid(P_R, P_1)
    r1 = r1 if sum(r1) else list(P_R)
    r2 = sampler.resid(P_2, P_1)
    Z1, Z2 = sum(r1), sum(r2)
    tot = Fraction(0)
    for x1, q in enumerate(law_sample(P_1)):
        if not q:
            continue
        rej = q * (1 - acc(P_R[x1], P_1[x1]))
        open_ = Z2 > 0 and (not gated or P_2[x1] < P_1[x1])
        if not open_:
            tot += rej
            continue
        for x2, q2 in enumerate(law_sample(r2)):
            if q2:
                tot += rej * q2 * (1 - acc(r1[x2] * Z2, Z1 * r2[x2]))
    return tot


@pytest.mark.parametrize("gated", [False, True])
def test_double_reject_bounds(gated):
    """Section 2.3: P(double reject) <= TV(p_d2, p_R) ungated, <= 2 TV(p_d2, p_R) gated."""
    for trial in range(30):
        V = 5
        ps = inputs.distributions(3, V, 5000 + trial, peaked=1.2)
        P_R, P_1, P_2 = (sampler.fixed(p) for p in ps)
        tv = 0.5 * sum(abs(a - b) for a, b in zip(P_2, P_R)) / float(1 << 40)
        pr = float(_double_reject_prob(P_R, P_1, P_2, gated))
        bound = (2 if gated else 1) * tv
        assert pr <= bound + 1e-9, (trial, pr, bound)


def _chi2_sf(x, k):
    from scipy.stats import chi2
    return float(chi2.sf(x, k))


@pytest.mark.parametrize("mode", list(MODES))
def test_cascade_chi_square_synthetic(mode):
    """10^5 seeded Philox draws through draw1/draw2/verify on fixed distributions chosen
    so every branch (first accept, second accept, double reject) is frequent."""
    V = 6
    p_R = np.array([0.30, 0.05, 0.25, 0.10, 0.20, 0.10], np.float32)
    p_1 = np.array([0.05, 0.40, 0.05, 0.30, 0.10, 0.10], np.float32)
    p_2 = np.array([0.10, 0.10, 0.40, 0.05, 0.05, 0.30], np.float32)
    P_R, P_1, P_2 = map(sampler.fixed, (p_R, p_1, p_2))
    N = 100_000
    counts = np.zeros(V)
    outcomes = np.zeros(5)
    for s in range(N):
        U = [philox.uniform(s, 17, k) for k in range(5)]
        x1 = sampler.draw1(P_1, U[0])
        gate, x2 = (False, -1)
        second, gated, residual = MODES[mode]
        if second:
            gate, x2 = sampler.draw2(P_1, P_2, x1, U[1], gated=gated, residual=residual)
        tok, out = sampler.verify(P_R, P_1, x1, U[2], U[4], gate, P_2, x2, U[3], residual=residual)
        counts[tok] += 1
        outcomes[out] += 1
    exp = p_R.astype(np.float64) / p_R.sum() * N
    stat = float(((counts - exp) ** 2 / exp).sum())
    assert _chi2_sf(stat, V - 1) > 1e-4, (stat, counts, exp)
    if mode != "single":
        assert outcomes[sampler.ACC2] > 1000 and outcomes[sampler.RESAMPLED] > 1000


def test_chi_square_detects_planted_reverification(monkeypatch):
    """A plausible mistake (re-verifying the second candidate against p_R instead of the
    residual target rho1) must be caught by the same statistic."""
    def bad_verify(P_R, P_d1, x1, U2, U4, gate_open=False, P_d2=None, x2=-1, U3=0):
        if sampler.accept(P_R, P_d1, x1, U2):
            return x1, sampler.ACC1
        r1 = sampler.resid(P_R, P_d1)
        if not gate_open:
            return sampler.sample(r1, U4), sampler.RESAMPLED
        r2 = sampler.resid(P_d2, P_d1)
        Z2 = sum(r2)
        if U3 * r2[x2] < ((P_R[x2] * Z2) << 32) // (1 << 40):   # wrong target p_R
            return x2, sampler.ACC2
        return sampler.sample(r1, U4), sampler.RESAMPLED

    V = 6
    p_R = np.array([0.30, 0.05, 0.25, 0.10, 0.20, 0.10], np.float32)
    p_1 = np.array([0.05, 0.40, 0.05, 0.30, 0.10, 0.10], np.float32)
    p_2 = np.array([0.10, 0.10, 0.40, 0.05, 0.05, 0.30], np.float32)
    P_R, P_1, P_2 = map(sampler.fixed, (p_R, p_1, p_2))
    N = 100_000
    counts = np.zeros(V)
    for s in range(N):
        U = [philox.uniform(s, 17, k) for k in range(5)]
        x1 = sampler.draw1(P_1, U[0])
        gate, x2 = sampler.draw2(P_1, P_2, x1, U[1], gated=False)
        tok, _ = bad_verify(P_R, P_1, x1, U[2], U[4], gate, P_2, x2, U[3])
        counts[tok] += 1
    exp = p_R.astype(np.float64) / p_R.sum() * N
    stat = float(((counts - exp) ** 2 / exp).sum())
    assert _chi2_sf(stat, V - 1) < 1e-6


def test_greedy_onehot_reduction():
    """One-hot readouts reduce the cascade to argmax comparisons (section 2.3)."""
    rnd = random.Random(3)
    V = 10
    for _ in range(200):
        a1, a2, aR = (rnd.randrange(V) for _ in range(3))
        oh = lambda a: [(1 << 40) if v == a else 0 for v in range(V)]
        P1, P2, PR = oh(a1), oh(a2), oh(aR)
        U = [rnd.randrange(1 << 32) for _ in range(5)]
        x1 = sampler.draw1(P1, U[0])
        assert x1 == a1
        gate, x2 = sampler.draw2(P1, P2, x1, U[1])
        assert gate == (a2 != a1) and (x2 == a2 if gate else x2 == -1)
        tok, out = sampler.verify(PR, P1, x1, U[2], U[4], gate, P2, x2, U[3])
        assert tok == aR
        assert out == (sampler.ACC1 if aR == a1 else sampler.ACC2 if (gate and aR == a2) else sampler.RESAMPLED)


def test_copy_cascade_law_and_order():
    """Point-mass cascade (q = delta_c in eq. 3-4): commits follow P_R exactly."""
    p_R = np.array([0.1, 0.4, 0.2, 0.3], np.float32)
    P_R = sampler.fixed(p_R)
    cands = [3, 1]
    N = 60_000
    counts = np.zeros(4)
    for s in range(N):
        Us = [philox.uniform(s, 9, philox.P_COPY0 + j) for j in range(2)]
        tok, out, j = sampler.verify_copy(P_R, cands, Us, philox.uniform(s, 9, philox.P_RESAMPLE))
        counts[tok] += 1
        if out == sampler.ACC_COPY:
            assert tok == cands[j]
    exp = p_R / p_R.sum() * N
    stat = float(((counts - exp) ** 2 / exp).sum())
    assert _chi2_sf(stat, 3) > 1e-4
