"""Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2,
3", SC'11), written from the published round function (test infrastructure only).

One round maps counter (c0, c1, c2, c3) with key (k0, k1) to
(hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)), where hi/lo are the
upper/lower 32 bits of the 64-bit product; the key is advanced by the Weyl constants
between rounds; ten rounds.

Uniform words consumed by the decoders: U(seed, pos, purpose) = word 0 of
Philox4x32-10 with key (seed mod 2^32, seed >> 32) and counter (pos, purpose, 0, 0).
They are keyed by the absolute position of the token being decided, so the committed
token at a position depends only on the committed prefix and these words.
Purposes: 0 first draw, 1 second draw, 2 first accept, 3 second accept, 4 residual
resample, 5 plain autoregressive draw, 8+j copy-candidate j.
"""

MASK = 0xFFFFFFFF
M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85

P_DRAW1, P_DRAW2, P_ACC1, P_ACC2, P_RESAMPLE, P_AR, P_COPY0 = 0, 1, 2, 3, 4, 5, 8


def philox4x32_10(ctr, key):
    c0, c1, c2, c3 = (int(x) & MASK for x in ctr)
    k0, k1 = (int(x) & MASK for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK, p1 & MASK, ((p0 >> 32) ^ c3 ^ k1) & MASK, p0 & MASK
    return c0, c1, c2, c3


def uniform(seed, pos, purpose):
    return philox4x32_10((pos, purpose, 0, 0), (seed & MASK, (seed >> 32) & MASK))[0]
