"""Pins of the oracle's confidence unmasking and denoising loop against closed
forms on hand-built logits, the pages' stated behaviour, invariants and brute
force."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_generation_defaults.json")


def _pages():
    with open(GOLDEN) as f:
        return json.load(f)


def _run(logits, masked=None, gamma=0.8, tau=1.0, mask_id=3, step=0, tokens=None):
    lg = np.asarray(logits, dtype=np.float64)
    B, S, V = lg.shape
    if masked is None:
        masked = np.ones((B, S), np.uint8)
    if tokens is None:
        tokens = np.where(np.asarray(masked) > 0, mask_id, 7)
    return oracle.confidence_unmask(lg, tokens, masked, gamma, tau, mask_id, step,
                                    commit_step=np.full((B, S), -1))


# U1 -- V = 2 with equal logits gives p = 1/2 exactly; the threshold is
# inclusive (gamma = 1/2 commits), and just above it nothing qualifies so the
# one-commit rule picks the lowest slot.
def test_u1_exact_half_and_inclusive_threshold():
    lg = np.zeros((1, 3, 2))
    r = _run(lg, gamma=0.5)
    assert np.all(r["conf"] == 0.5)
    assert r["committed_now"].tolist() == [[1, 1, 1]]
    assert r["pred"].tolist() == [[0, 0, 0]]
    r = _run(lg, gamma=0.5 + 2.0 ** -20)
    assert r["committed_now"].tolist() == [[1, 0, 0]]
    assert r["tokens"].tolist() == [[0, 3, 3]]
    assert r["n_masked"].tolist() == [2]


# U2 -- one logit a and V-1 zeros: p = e^a / (e^a + V - 1); a chosen for p = 0.9
# (commits at gamma 0.8) and p = 0.7 (does not).
@pytest.mark.parametrize("V", [16, 1024, 131072])
def test_u2_planted_logit_closed_form(V):
    def a_for(p):
        return math.log(p * (V - 1) / (1 - p))
    lg = np.zeros((1, 2, V))
    lg[0, 0, 5] = a_for(0.9)
    lg[0, 1, V - 1] = a_for(0.7)
    r = _run(lg, gamma=0.8)
    for s, (a, idx) in enumerate([(a_for(0.9), 5), (a_for(0.7), V - 1)]):
        expect = math.exp(a) / (math.exp(a) + V - 1)
        assert abs(r["conf"][0, s] - expect) < 1e-14
        assert r["pred"][0, s] == idx
    assert r["committed_now"].tolist() == [[1, 0]]
    assert r["tokens"].tolist() == [[5, 3]]


# U3 -- all rows below gamma: exactly one commit, at the largest p; identical
# rows: the lowest slot.
def test_u3_one_commit_rule():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((1, 6, 64)) * 0.1          # p ~ 1/64 everywhere
    lg[0, 4, 10] = 2.0                                   # slot 4 most confident
    r = _run(lg, gamma=0.8)
    assert r["committed_now"].sum() == 1 and r["committed_now"][0, 4] == 1
    assert r["tokens"][0, 4] == 10
    same = np.tile(lg[:, :1], (1, 6, 1))
    masked = np.array([[0, 1, 1, 1, 1, 1]], np.uint8)    # slot 0 already committed
    r = _run(same, masked=masked, gamma=0.8)
    assert r["committed_now"].tolist() == [[0, 1, 0, 0, 0, 0]]
    assert r["tokens"][0, 0] == 7                        # untouched committed slot


# U4 -- ties in the logits: the lowest token id wins.
def test_u4_lowest_id_on_ties():
    lg = np.zeros((1, 2, 10))
    lg[0, 0, [7, 2, 9]] = 4.0
    lg[0, 1, [9, 8]] = 4.0
    r = _run(lg, gamma=0.0)
    assert r["pred"].tolist() == [[2, 8]]


# U5 / U8 -- loop invariants on random logits, with the pages' constants:
# a block with n masked slots finishes within n steps, every step commits at
# least one slot, committed tokens never change, n_masked strictly decreases,
# and S = steps_per_block steps always suffice.
@pytest.mark.parametrize("seed", range(4))
def test_u5_u8_loop_invariants(seed):
    pg = _pages()
    S, V = pg["block_size"], 50
    assert pg["steps_per_block"] == S
    rng = np.random.default_rng(seed)
    B = 3
    masked = (rng.random((B, S)) < 0.7).astype(np.uint8)
    masked[0] = 1
    tokens = np.where(masked > 0, pg["mask_token_id"], rng.integers(0, V, (B, S)))
    n0 = masked.sum(1)
    step_logits = {k: rng.standard_normal((B, S, V)) * 3 for k in range(S)}
    q = np.zeros((B, S, 1, 4))
    kv = np.zeros((B, S, 1, 4))
    ctx = np.zeros((1, 1, 4))
    r = oracle.denoise_block(lambda k, l: (q, kv, kv), lambda k: step_logits[k],
                             [ctx], [ctx], np.zeros(B, np.int64), np.zeros(B, np.int32),
                             tokens, masked, pg["confidence_threshold"],
                             pg["temperature"], pg["mask_token_id"],
                             max_steps=pg["steps_per_block"])
    tr = r["n_masked_trace"]
    assert r["masked"].sum() == 0
    assert r["steps_taken"] <= n0.max()
    for b in range(B):
        for k in range(1, tr.shape[0]):
            if tr[k - 1, b] > 0:
                assert tr[k, b] < tr[k - 1, b]
            else:
                assert tr[k, b] == 0
        keep = masked[b] == 0
        np.testing.assert_array_equal(r["tokens"][b][keep], tokens[b][keep])
        assert np.all(r["commit_step"][b][keep] == -1)
        assert np.all(r["commit_step"][b][~keep] >= 0)
    # replay the steps one by one: once committed a token never changes
    tok, msk = tokens.copy(), masked.copy()
    for k in range(r["steps_taken"]):
        st = oracle.confidence_unmask(step_logits[k], tok, msk, 0.8, 0.1, 3, k)
        fixed = msk == 0
        assert np.array_equal(st["tokens"][fixed], tok[fixed])
        tok, msk = st["tokens"], st["masked"]
    np.testing.assert_array_equal(tok, r["tokens"])


# U6 -- monotone in gamma ([dothoosh] benchmark paragraph: a lower threshold
# commits more tokens per step): commit set at gamma1 contains that at gamma2.
def test_u6_monotone_in_gamma():
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((4, 16, 256)) * 3.0
    sets = []
    for g in [0.3, 0.6, 0.8, 0.95]:
        r = _run(lg, gamma=g)
        sets.append(r["committed_now"].astype(bool))
    for lo, hi in zip(sets, sets[1:]):
        # every slot committed at the higher gamma is committed at the lower
        # one (the one-commit fallback picks the top slot, which any
        # non-empty threshold set contains)
        assert np.all(lo | ~hi)
    counts = [s.sum() for s in sets]
    assert counts == sorted(counts, reverse=True)
    assert counts[0] > counts[-1]


# U7 -- V = 2, logits (a, 0): p = 1 / (1 + e^(-a/tau)) for several tau,
# including the pages' tau = 0.1.
@pytest.mark.parametrize("tau", [0.1, 0.5, 1.0, 2.0])
def test_u7_temperature_closed_form(tau):
    a = np.array([0.05, 0.3, -0.2, 1.0])
    lg = np.stack([np.stack([a, np.zeros_like(a)], -1)])       # [1, 4, 2]
    r = _run(lg, gamma=0.99, tau=tau)
    for s in range(4):
        expect = 1.0 / (1.0 + math.exp(-abs(a[s]) / tau))
        assert abs(r["conf"][0, s] - expect) < 1e-15
        assert r["pred"][0, s] == (0 if a[s] >= 0 else 1)


# R16 -- the mask id may be predicted: the slot commits with token 3 and its
# mask bit clears; the uncommitted masked slots are written as the mask id.
def test_mask_id_prediction_commits():
    lg = np.full((1, 3, 8), -5.0)
    lg[0, 0, 3] = 10.0
    r = _run(lg, gamma=0.8, tokens=np.array([[3, 6, 6]]))
    assert r["tokens"].tolist() == [[3, 3, 3]]
    assert r["masked"].tolist() == [[0, 1, 1]]
    assert r["commit_step"].tolist() == [[0, -1, -1]]


def test_nothing_masked_is_a_noop():
    lg = np.random.default_rng(0).standard_normal((2, 4, 8))
    masked = np.zeros((2, 4), np.uint8)
    tokens = np.arange(8).reshape(2, 4)
    r = _run(lg, masked=masked, tokens=tokens)
    np.testing.assert_array_equal(r["tokens"], tokens)
    assert r["committed_now"].sum() == 0 and r["n_masked"].tolist() == [0, 0]
    assert np.all(np.isnan(r["conf"])) and np.all(r["pred"] == -1)


# U9 -- brute force: a scalar-loop restatement with its own softmax (a full
# probability vector normalised by a plain sum) on tiny shapes.
def _brute(lg, masked, gamma, tau):
    B, S, V = lg.shape
    out = []
    for b in range(B):
        ps = {}
        for s in range(S):
            if not masked[b][s]:
                continue
            row = [lg[b][s][v] / tau for v in range(V)]
            mx = row[0]
            arg = 0
            for v in range(1, V):
                if row[v] > mx:
                    mx, arg = row[v], v
            w = [math.exp(x - mx) for x in row]
            tot = sum(w)
            ps[s] = (arg, w[arg] / tot)
        com = sorted(s for s in ps if ps[s][1] >= gamma)
        if not com and ps:
            best = max(p for _, p in ps.values())
            com = [min(s for s in ps if ps[s][1] == best)]
        out.append((com, {s: ps[s][0] for s in ps}))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_u9_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    B, S, V = 3, 4, 8
    lg = np.round(rng.standard_normal((B, S, V)) * 2, 1)
    masked = (rng.random((B, S)) < 0.8).astype(np.uint8)
    gamma, tau = [0.5, 0.8, 0.3][seed % 3], [1.0, 0.1, 0.5][seed % 3]
    r = _run(lg, masked=masked, gamma=gamma, tau=tau)
    for b, (com, preds) in enumerate(_brute(lg, masked, gamma, tau)):
        assert sorted(np.flatnonzero(r["committed_now"][b]).tolist()) == com
        for s, v in preds.items():
            assert r["pred"][b, s] == v
            if s in com:
                assert r["tokens"][b, s] == v
            else:
                assert r["tokens"][b, s] == 3
    assert r["ambiguous"] == 0


def test_pages_defaults_fixture():
    pg = _pages()
    assert (pg["block_size"], pg["steps_per_block"], pg["mask_token_id"]) == (16, 16, 3)
    assert pg["confidence_threshold"] == 0.8 and pg["temperature"] == 0.1
    assert pg["max_new_tokens"] % pg["block_size"] == 0
