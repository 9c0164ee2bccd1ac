"""Copy-suffix proposals with shallow screening (test infrastructure only).

CopyLoop page (kongchang.com, "CopyLoop"): candidate continuations are copied from
repeated context at almost no cost, scored at a shallow loop depth, and low scorers are
dropped before full-depth verification; the threshold is set by light calibration.  The
page gives no concrete rule, so this is one reading (it affects speed only: any
candidate set that does not depend on the verification uniforms keeps the committed
distribution equal to p_R):

* candidates(prefix): for n = 3, 2, 1, take the occurrences of the last n tokens earlier
  in the prefix, most recent first; their following tokens, de-duplicated in order of
  discovery, are the candidates; the longest n with any match wins; at most 16.
* screening: candidate c survives iff A_s(c) >= floor(tau * 2^40), with A_s the fixed-point
  readout at the screening depth s.  Survivors are ordered by A_s descending, then id.
"""

SHIFT = 40


def candidates(prefix, max_cands=16):
    toks = list(prefix)
    L = len(toks)
    for n in (3, 2, 1):
        if L <= n:
            continue
        suf = toks[L - n:]
        out = []
        for i in range(L - 1, n - 1, -1):          # continuation index i, match toks[i-n:i]
            if toks[i - n:i] == suf and toks[i] not in out:
                out.append(toks[i])
                if len(out) == max_cands:
                    break
        if out:
            return out
    return []


def screen(cands, A_s, tau):
    thr = int(tau * (1 << SHIFT))
    surv = [c for c in cands if A_s[c] >= thr]
    surv.sort(key=lambda c: (-A_s[c], c))
    return surv
