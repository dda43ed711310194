"""Counter-based random numbers and temperature sampling for unmasking
(test infrastructure; see the package header).

Pages followed (tags defined in oracle/__init__.py):
  * [news] "training and inference" code example: the generation call takes
    a temperature (0.1 in the example) next to the confidence threshold.
  * [keyframe] "key points" item 3: all masked slots are predicted at once and
    the confident ones are committed.

Readings where the pages are silent:
  * temperature sampling draws the prediction of a masked slot from
    softmax(l / tau) with the Gumbel-max rule: x = argmax_v (l_v / tau + G_v),
    G_v iid standard Gumbel, lowest v on ties; since tau > 0 this is the same
    argmax as that of l_v + tau * G_v;
  * the confidence of the slot is the probability of the drawn token under
    the distribution it was drawn from, softmax(l / tau)[x]; the commit rule
    is unchanged;
  * G_v comes from the counter-based generator Philox4x32-10 (J. K. Salmon,
    M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as
    1, 2, 3", SC 2011): key = the 64-bit seed (low word first), counter =
    (v // 4, b * S + s, step, block), word v % 4 of the output; the word w
    becomes u = (2 * (w >> 9) + 1) / 2^24 (23 random bits, u in (0, 1),
    exactly representable in fp32 and fp64) and G = -ln(-ln u).
"""

import math

import numpy as np

_MASK32 = np.uint64(0xFFFFFFFF)
# Philox4x32 round multipliers and Weyl key increments (Salmon et al., 2011)
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.  counter: 4 sequences of uint32 values (each
    an int or an array; they broadcast), key: 2 uint32 values.  Each round
    takes the two 64-bit products M0*c0 and M1*c2, and forms the next counter
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
    is bumped by the Weyl constants between rounds.  Returns 4 uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in counter]
    c = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = (np.array(x, dtype=np.uint64) for x in c)
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = _M0 * c0            # < 2^64: exact in uint64
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return [x.astype(np.uint32) for x in (c0, c1, c2, c3)]


def uniform_words(seed, row_id, step, block, V):
    """The V uniforms of one slot: word v % 4 of Philox4x32-10 at counter
    (v // 4, row_id, step, block) with key (seed low, seed high), mapped to
    u = (2 * (w >> 9) + 1) / 2^24."""
    seed = int(seed)
    n = (V + 3) // 4
    out = philox4x32_10((np.arange(n, dtype=np.uint64), row_id, step, block),
                        (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    w = np.stack(out, axis=1).reshape(-1)[:V].astype(np.uint64)
    return (2.0 * (w >> np.uint64(9)).astype(np.float64) + 1.0) / 16777216.0


def gumbel_noise(seed, row_id, step, block, V):
    """G_v = -ln(-ln u_v) in fp64 for the V tokens of one slot."""
    u = uniform_words(seed, row_id, step, block, V)
    return -np.log(-np.log(u))


def row_sample(row, temperature, seed, row_id, step, block):
    """(pred, p, margin) for one logit row under temperature sampling:
    pred = lowest argmax_v (l_v + tau * G_v); p = exp((l_pred - m) / tau) / Z
    with m = max l and Z = sum_v exp((l_v - m) / tau) (exactly rounded sum);
    margin = gap between the best and the second-best perturbed score (inf
    for a one-token vocabulary)."""
    x = np.asarray(row, dtype=np.float64)
    tau = float(temperature)
    g = gumbel_noise(seed, row_id, step, block, x.shape[0])
    key = x + tau * g
    best = key.max()
    pred = int(np.flatnonzero(key == best)[0])
    rest = np.delete(key, pred)
    margin = float(best - rest.max()) if rest.size else math.inf
    m = x.max()
    z = math.fsum(np.exp((x - m) / tau).tolist())
    return pred, math.exp((x[pred] - m) / tau) / z, margin
