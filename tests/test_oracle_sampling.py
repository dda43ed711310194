"""Pins of the oracle's counter-based generator and temperature sampling
against published known answers, distributional facts and closed forms --
never against the oracle's own formula retyped."""
import math

import numpy as np

import oracle
from oracle import sampling


# S1 -- Philox4x32-10 known-answer vectors published with the generator
# (Salmon et al., SC 2011; the Random123 distribution's known-answer tests):
# zero counter and key, all-ones counter and key, and the pi-digits case.
def test_s1_philox_known_answers():
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in cases:
        got = tuple(int(x) for x in sampling.philox4x32_10(ctr, key))
        assert got == want, (ctr, key, [hex(x) for x in got])
    # vectorised counters give the same words as one-at-a-time calls
    v = sampling.philox4x32_10((np.arange(5), 7, 1, 2), (11, 13))
    for i in range(5):
        one = sampling.philox4x32_10((i, 7, 1, 2), (11, 13))
        assert [int(x[i]) for x in v] == [int(x) for x in one]


# S2 -- the uniform map: 23 random bits, u = (2k + 1) / 2^24 strictly inside
# (0, 1), exactly representable in fp32; the extreme words map to 2^-24 and
# 1 - 2^-24.
def test_s2_uniform_map():
    u = sampling.uniform_words(12345, 3, 0, 0, 4096)
    assert u.min() > 0.0 and u.max() < 1.0
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    k = u * 2 ** 24
    assert np.array_equal(k, np.round(k)) and np.all(k % 2 == 1)
    # word of v = 0: take it from the generator itself and map by hand
    w0 = int(sampling.philox4x32_10((0, 3, 0, 0), (12345, 0))[0])
    assert u[0] == (2 * (w0 >> 9) + 1) / 2 ** 24


# S3 -- Gumbel noise moments: mean = Euler-Mascheroni constant, variance =
# pi^2 / 6 (standard Gumbel), within 6 standard errors over 2^20 draws.
def test_s3_gumbel_moments():
    g = np.concatenate([sampling.gumbel_noise(7, r, 0, 0, 1 << 16) for r in range(16)])
    n = g.size
    mean_se = math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.mean() - 0.5772156649015329) < 6 * mean_se
    # the variance of a Gumbel sample variance: (mu4 - sigma^4)/n, mu4 = 27/5 sigma^4
    var = math.pi ** 2 / 6
    var_se = math.sqrt((5.4 - 1.0) * var ** 2 / n)
    assert abs(g.var() - var) < 6 * var_se


# S4 -- the Gumbel-max rule samples from softmax(l / tau): over many slots
# (row ids) the frequency of each token matches its probability within 6
# binomial standard errors, for two temperatures.
def test_s4_sampling_follows_softmax():
    l = np.array([1.0, 0.5, 0.0, -1.0, 2.0])
    for tau in (1.0, 0.5):
        p = np.exp(l / tau - (l / tau).max())
        p /= p.sum()
        n = 20000
        counts = np.zeros(5)
        for r in range(n):
            pred, _, _ = sampling.row_sample(l, tau, 99, r, 0, 0)
            counts[pred] += 1
        se = np.sqrt(p * (1 - p) / n)
        assert np.all(np.abs(counts / n - p) < 6 * se), (tau, counts / n, p)


# S5 -- closed forms: the reported confidence is softmax(l/tau) at the drawn
# token; with two tokens it is the logistic of their gap; far-apart logits
# (gap beyond tau times the noise range) make sampling the argmax, with the
# greedy confidence.
def test_s5_confidence_closed_forms():
    for r in range(50):
        pred, p, _ = sampling.row_sample([0.3, -0.4], 0.7, 5, r, 2, 1)
        gap = (0.3 - -0.4) if pred == 0 else (-0.4 - 0.3)
        assert abs(p - 1.0 / (1.0 + math.exp(-gap / 0.7))) < 1e-15
    rng = np.random.default_rng(0)
    row = rng.standard_normal(1000)
    row[417] = row.max() + 25.0             # 25 > 0.1 * (16.64 + 2.82)
    for r in range(20):
        pred, p, _ = sampling.row_sample(row, 0.1, 1, r, 0, 0)
        g_pred, g_p = oracle.row_confidence(row, 0.1)
        assert pred == 417 == g_pred and p == g_p


# S6 -- counter independence: the noise depends on every counter field and
# on both seed words, and repeats exactly for the same inputs.
def test_s6_counter_fields():
    base = sampling.gumbel_noise(5, 1, 2, 3, 64)
    assert np.array_equal(base, sampling.gumbel_noise(5, 1, 2, 3, 64))
    for args in [(6, 1, 2, 3), (5, 2, 2, 3), (5, 1, 3, 3), (5, 1, 2, 4), (5 + (1 << 32), 1, 2, 3)]:
        other = sampling.gumbel_noise(*args, 64)
        assert np.mean(other == base) < 0.05, args


# S7 -- the sampled unmasking pass keeps the commit rule: a hand-built batch
# where every slot's drawn token is forced (huge logit gap) commits exactly
# the slots whose p reaches gamma; the one-commit rule and commit_all hold.
def test_s7_sampled_unmask_commit_rule():
    B, S, V = 2, 4, 8
    lg = np.zeros((B, S, V))
    lg[0, :, 2] = 40.0                       # p ~ 1 at tau = 1: all commit
    lg[1, :, :] = 0.0                        # uniform: p = 1/8 each, one commit
    lg[1, 2, 5] = 0.5                        # slot 2's p can be the largest
    tok = np.full((B, S), 3)
    msk = np.ones((B, S), np.uint8)
    r = oracle.confidence_unmask(lg, tok, msk, 0.8, 1.0, 3, 0, sample=(17, 0))
    assert r["committed_now"][0].tolist() == [1, 1, 1, 1]
    assert r["tokens"][0].tolist() == [2, 2, 2, 2]
    assert r["committed_now"][1].sum() == 1
    best = int(np.argmax(r["conf"][1]))
    assert r["committed_now"][1, best] == 1
    for s in range(S):                       # conf = softmax at the drawn token
        x = lg[1, s]
        e = np.exp(x - x.max())
        assert abs(r["conf"][1, s] - e[r["pred"][1, s]] / e.sum()) < 1e-15
    r2 = oracle.confidence_unmask(lg, tok, msk, 0.8, 1.0, 3, 0, sample=(17, 0), commit_all=True)
    assert r2["masked"].sum() == 0 and np.array_equal(r2["pred"], r["pred"])
