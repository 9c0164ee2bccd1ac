"""Readout distribution of C (test infrastructure only).

LoopSpec page, section 2.1: C includes temperature scaling, an optional truncation and
normalisation, and every intermediate readout applies the same processing as the
target.  Order used here: temperature, softmax, top-p truncation, renormalisation.

Readings where the page is silent: top-p keeps the tokens of highest probability, ties
ordered by ascending id, up to and including the first token at which the kept mass
reaches top_p (a token is kept iff the mass strictly before it is below top_p);
top_p >= 1 keeps every token; greedy decoding is the one-hot distribution at the argmax
(lowest id on ties).
"""

import numpy as np


def greedy_onehot(logits):
    lg = np.asarray(logits, np.float64)
    p = np.zeros(lg.shape[0], np.float32)
    p[int(np.argmax(lg))] = 1.0          # np.argmax returns the first (lowest) index on ties
    return p


def softmax_t(logits, T):
    z = np.asarray(logits, np.float64) / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def top_p_keep(p, top_p):
    """Boolean mask of the tokens kept by top-p truncation of the float64 distribution p."""
    V = p.shape[0]
    if top_p >= 1.0:
        return np.ones(V, bool)
    order = np.lexsort((np.arange(V), -p))           # p descending, then id ascending
    before = np.concatenate([[0.0], np.cumsum(p[order])[:-1]])
    keep = np.zeros(V, bool)
    keep[order[before < top_p]] = True
    return keep


def distribution(logits, greedy, T=1.0, top_p=1.0):
    """float32 probability vector of the processed readout."""
    if greedy:
        return greedy_onehot(logits)
    p = softmax_t(logits, T)
    keep = top_p_keep(p, top_p)
    q = np.where(keep, p, 0.0)
    q = q / q.sum()
    return q.astype(np.float32)
