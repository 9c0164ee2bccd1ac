"""Lossless verification in integer fixed point (test infrastructure only).

LoopSpec page, section 2.2 and 2.3:
* eq. 2, residual operator: (mu (-) nu)(v) = [mu(v) - nu(v)]_+ / sum_u [mu(u) - nu(u)]_+;
  a zero denominator means mu = nu and the rejection event has probability zero.
* eq. 3-4, single candidate: x~ ~ q, accept with min(1, p(x~)/q(x~)), otherwise draw
  x ~ p (-) q.
* eq. 5-6, second proposal q2 = p_d2 (-) p_d1, drawn only when the gate is open:
  p_d2(x~1) < p_d1(x~1).
* Table 3 (section 3.4) ablates the residual form: the non-residual second proposal is
  p_d2 with the first candidate removed and renormalised; everything after it (the
  cascade below, with this q2) is unchanged, and it stays lossless because after x~1 is
  rejected the target is rho1 whatever distribution x~2 came from.
* cascade: rho1 = p_R (-) q1; the second candidate is accepted with
  min(1, rho1(x~2)/q2(x~2)); after two rejections x ~ rho1 (-) q2; with the gate closed
  the first rejection draws from rho1.  The second candidate is never re-verified against
  p_R itself.

Fixed point (a reading; the page gives real-number formulas): a float32 probability p
becomes the integer A = floor(p * 2^40).  Every step below is then exact integer
arithmetic on Python ints, so identical inputs give identical decisions:
  SAMPLE(A, U): Z = sum(A), t = floor(U * Z / 2^32), return the smallest v whose
                prefix sum A(0) + ... + A(v) exceeds t.     (inverse CDF, U in [0, 2^32))
  ACCEPT(P, Q, x, U):  U * Q(x) < P(x) * 2^32               (U/2^32 < P(x)/Q(x))
  RESID(A, B) = max(0, A - B) elementwise                    (numerator of eq. 2)
A residual that is all zero after quantisation falls back to the distribution it was
taken from (rho1 := p_R; rho1 (-) q2 := rho1; a zero q2 closes the gate).
"""

SHIFT = 40
ONE = 1 << SHIFT

ACC1, ACC2, RESAMPLED, DRAWN = 1, 2, 3, 4
ACC_COPY = 5          # a copy candidate accepted


def fixed(p):
    """float32 probabilities -> list of ints floor(p * 2^40) (exact: p has 24 bits)."""
    import numpy as np
    a = np.floor(np.asarray(p, np.float32).astype(np.float64) * float(ONE))
    return [int(x) for x in a]


def sample(A, U):
    Z = sum(A)
    if Z <= 0:
        raise ValueError("SAMPLE on an all-zero vector")
    t = (U * Z) >> 32
    c = 0
    for v, a in enumerate(A):
        c += a
        if c > t:
            return v
    raise AssertionError("unreachable")


def accept(P, Q, x, U):
    return U * Q[x] < (P[x] << 32)


def resid(A, B):
    return [a - b if a > b else 0 for a, b in zip(A, B)]


def draw1(P_d1, U0):
    """First proposal x~1 ~ q1 = p_d1."""
    return sample(P_d1, U0)


def proposal2(P_d1, P_d2, x1, residual=True):
    """Unnormalised second proposal: the residual p_d2 (-) p_d1 of eq. 5, or (residual=False,
    Table 3's non-residual ablation) p_d2 with the first candidate x1 masked to zero."""
    if residual:
        return resid(P_d2, P_d1)
    r = list(P_d2)
    r[x1] = 0
    return r


def draw2(P_d1, P_d2, x1, U1, gated=True, residual=True):
    """Gate (eq. 6) and second proposal (eq. 5).  Returns (gate_open, x2 or -1)."""
    r2 = proposal2(P_d1, P_d2, x1, residual)
    if sum(r2) == 0:
        return False, -1
    if gated and not (P_d2[x1] < P_d1[x1]):
        return False, -1
    return True, sample(r2, U1)


def verify(P_R, P_d1, x1, U2, U4, gate_open=False, P_d2=None, x2=-1, U3=0, residual=True):
    """Cascade verification at full depth.  Returns (token, outcome)."""
    if accept(P_R, P_d1, x1, U2):
        return x1, ACC1
    r1 = resid(P_R, P_d1)
    if sum(r1) == 0:
        r1 = list(P_R)
    if not gate_open:
        return sample(r1, U4), RESAMPLED
    r2 = proposal2(P_d1, P_d2, x1, residual)
    Z1, Z2 = sum(r1), sum(r2)
    # accept x~2 with probability min(1, rho1(x2) / q2(x2)), rho1 = r1/Z1, q2 = r2/Z2
    if U3 * Z1 * r2[x2] < ((r1[x2] * Z2) << 32):
        return x2, ACC2
    r3 = [a * Z2 - b * Z1 for a, b in zip(r1, r2)]
    r3 = [x if x > 0 else 0 for x in r3]
    if sum(r3) == 0:
        r3 = r1
    return sample(r3, U4), RESAMPLED


def verify_copy(P_R, cands, Us, U4):
    """Point-mass cascade over distinct deterministic candidates c_1..c_k (eq. 3-4 with
    q = delta_c, applied in order; each rejection removes c_j from the target).
    Returns (token, outcome, j) with j the accepted candidate's index or -1."""
    rho = list(P_R)
    for j, c in enumerate(cands):
        Z = sum(rho)
        if Us[j] * Z < (rho[c] << 32):
            return c, ACC_COPY, j
        rho[c] = 0
    return sample(rho, U4), RESAMPLED, -1
