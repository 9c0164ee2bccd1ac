"""Copy-suffix candidates and shallow screening for the scheduler (CopyLoop page:
candidates copied from repeated context, scored at a shallow loop depth, low scorers
dropped before full-depth verification; the threshold needs light calibration).

The rule (which tokens, in which order) must be a function of the prefix alone, so that
the pipelined decoder verifies the same candidates a serial decoder would; the rule itself
only affects speed.  Here: the longest n in {3, 2, 1} for which the last n tokens occurred
earlier; the tokens that followed those occurrences, most recent occurrence first, without
repeats, at most `max_cands`.  Screening (on the device, ls_verify's SCREEN job) keeps c when
floor(p_s(c) * 2^40) >= floor(tau * 2^40) and orders survivors by that value (descending),
then by token id.
"""

import numpy as np


def candidates(prefix, max_cands=16):
    seq = np.asarray(prefix, dtype=np.int64)
    n_tok = len(seq)
    for n in (3, 2, 1):
        if n_tok <= n:
            continue
        tail = seq[n_tok - n:]
        # windows seq[i-n:i] for i = n .. n_tok-1 (i = index of the following token)
        win = np.lib.stride_tricks.sliding_window_view(seq[:n_tok - 1], n)      # starts 0 .. n_tok-1-n
        hits = np.nonzero((win == tail).all(axis=1))[0] + n                      # following-token index
        if hits.size == 0:
            continue
        out, seen = [], set()
        for i in hits[::-1]:
            t = int(seq[i])
            if t not in seen:
                seen.add(t)
                out.append(t)
                if len(out) == max_cands:
                    break
        return out
    return []


def threshold(tau):
    """Fixed-point screening threshold floor(tau * 2^40): candidate c survives when
    floor(p_s(c) * 2^40) reaches it (the device screening job compares in that fixed point)."""
    return int(tau * float(1 << 40))
