"""Pins of the oracle's multi-block generation loop on hand-built providers:
stop rules, what the caches hold afterwards, state carried from one block to
the next (checked through the separately pinned attention), and the
final-step rule."""
import numpy as np

import oracle

RNG = np.random.default_rng

B, S, Hq, Hkv, d, V, NL = 3, 4, 4, 2, 8, 16, 2
EOS, MASK = 9, 3


def _setup(lens=(5, 0, 3), room=3, seed=0):
    r = RNG(seed)
    cap = [l + room * S for l in lens]
    start = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    end = start + np.asarray(cap)
    T = int(sum(cap))
    kc = [r.standard_normal((T, Hkv, d)) for _ in range(NL)]
    vc = [r.standard_normal((T, Hkv, d)) for _ in range(NL)]
    den = {}
    ctx = {}

    def denoise_inputs(blk, k, l):
        key = (blk, k, l)
        if key not in den:
            rr = RNG(1000 + 100 * blk + 10 * k + l)
            den[key] = (rr.standard_normal((B, S, Hq, d)), rr.standard_normal((B, S, Hkv, d)),
                        rr.standard_normal((B, S, Hkv, d)))
        return den[key]

    def ctx_inputs(blk, l, tokens):
        key = (blk, l)
        if key not in ctx:
            rr = RNG(5000 + 10 * blk + l)
            # the provider's K/V depend on the committed tokens (an embedding)
            emb = np.asarray(tokens, dtype=np.float64)[..., None, None] / 10.0
            ctx[key] = (rr.standard_normal((B, S, Hq, d)),
                        rr.standard_normal((B, S, Hkv, d)) + emb,
                        rr.standard_normal((B, S, Hkv, d)) - emb)
        return ctx[key]
    return dict(start=start, end=end, lens=np.asarray(lens), kc=kc, vc=vc,
                denoise_inputs=denoise_inputs, ctx_inputs=ctx_inputs, den=den, ctx=ctx)


def _logits_eos_first_block(blk, k):
    """Every slot confident (one dominant logit); sequence 0 predicts EOS at
    slot 2 of block 0, everything else predicts token 5 + slot."""
    lg = np.zeros((B, S, V))
    for s in range(S):
        lg[:, s, 5 + s] = 30.0
    if blk == 0:
        lg[0, 2, :] = 0.0
        lg[0, 2, EOS] = 30.0
    return lg


def _run(st, logits_fn, n_blocks=3, **kw):
    return oracle.generate(st["denoise_inputs"], logits_fn, st["ctx_inputs"], st["kc"], st["vc"],
                           st["start"], st["end"], st["lens"], S, n_blocks, 0.8, 1.0, MASK,
                           eos_token_id=EOS, **kw)


# G1 -- EOS stop: sequence 0 commits EOS in block 0 and stops there; the
# others run every block.  Tokens, counts and stop reasons by hand.
def test_g1_eos_stop():
    st = _setup()
    r = _run(st, _logits_eos_first_block)
    assert r["blocks_taken"] == 3
    assert r["stop"].tolist() == [1, 0, 0]
    assert r["n_generated"].tolist() == [S, 3 * S, 3 * S]
    assert r["tokens"][0, :S].tolist() == [5, 6, EOS, 8] and np.all(r["tokens"][0, S:] == -1)
    for b in (1, 2):
        assert r["tokens"][b].tolist() == [5, 6, 7, 8] * 3
    assert r["ctx_len"].tolist() == [5 + S, 3 * S, 3 + 3 * S]
    # every block was final after one step (all slots confident)
    assert all(x["steps_taken"] == 1 for x in r["denoise"])


# G2 -- the caches afterwards: each sequence's region holds its context, then
# the context tower's K/V of each block it generated, in order; nothing else
# changed.
def test_g2_cache_contents():
    st = _setup()
    kc0 = [x.copy() for x in st["kc"]]
    r = _run(st, _logits_eos_first_block)
    for l in range(NL):
        want = kc0[l].copy()
        for b in range(B):
            pos = int(st["start"][b]) + int(st["lens"][b])
            for blk in range(r["n_generated"][b] // S):
                want[pos:pos + S] = st["ctx"][(blk, l)][1][b]
                pos += S
        np.testing.assert_array_equal(r["k_ctx"][l], want)


# G3 -- state carried across blocks: the denoiser's first-step attention in
# block 1 equals attention over the explicit concatenation [context ; block-0
# K/V of the context tower], and the context tower's attention in block 1
# is causal attention over [context ; block 0 ; block 1].
def test_g3_next_block_sees_committed_block():
    st = _setup()
    kc0 = [x.copy() for x in st["kc"]]
    vc0 = [x.copy() for x in st["vc"]]
    r = _run(st, _logits_eos_first_block, n_blocks=2)
    for l in range(NL):
        q, kb, vb = st["den"][(1, 0, l)]
        out1, _ = r["denoise"][1]["outputs"][0][l]
        c_out, _ = r["ctx_outputs"][1][l]
        for b in (1, 2):
            st_b, n = int(st["start"][b]), int(st["lens"][b])
            kcat = np.concatenate([kc0[l][st_b:st_b + n], st["ctx"][(0, l)][1][b]], axis=0)
            vcat = np.concatenate([vc0[l][st_b:st_b + n], st["ctx"][(0, l)][2][b]], axis=0)
            ref, _ = oracle.block_attn(q[b:b + 1], kb[b:b + 1], vb[b:b + 1], kcat, vcat,
                                       np.array([0]), np.array([n + S]))
            np.testing.assert_allclose(out1[b], ref[0], rtol=0, atol=1e-12)
            cq, ck, cv = st["ctx"][(1, l)]
            cref, _ = oracle.ctx_block_attn(cq[b:b + 1], ck[b:b + 1], cv[b:b + 1], kcat, vcat,
                                            np.array([0]), np.array([n + S]))
            np.testing.assert_allclose(c_out[b], cref[0], rtol=0, atol=1e-12)
        assert np.isnan(out1[0]).all()        # sequence 0 stopped: no rows


# G4 -- finality: with nothing confident and steps_per_block < S, the one-
# commit rule commits one slot per step and the last allowed step commits the
# rest, so every generated slot holds a token and no mask id is left.
def test_g4_last_step_commits_the_rest():
    st = _setup()

    def flat(blk, k):
        lg = np.zeros((B, S, V))
        lg[:, :, 4] = 1.0                    # p = e/(e+15) < 0.8: never confident
        return lg
    r = _run(st, flat, n_blocks=2, steps_per_block=2)
    for x in r["denoise"]:
        assert x["steps_taken"] == 2
        assert x["n_masked_trace"].tolist() == [[S] * B, [S - 1] * B, [0] * B]
    assert np.all(r["tokens"] == 4) and r["stop"].tolist() == [0, 0, 0]


# G5 -- cache room: a region with room for one block only stops the sequence
# after it (stop = 2); its length grew once.
def test_g5_room_stop():
    st = _setup(room=3)
    st["end"] = st["end"].copy()
    for b in (0, 2):                          # room for one block only
        st["end"][b] = st["start"][b] + st["lens"][b] + S
    r = _run(st, lambda blk, k: _logits_eos_first_block(1, k), n_blocks=3)
    assert r["stop"].tolist() == [2, 0, 2]
    assert r["n_generated"].tolist() == [2 * S, 3 * S, 2 * S]
    assert r["ctx_len"].tolist() == [5 + S, 3 * S, 3 + S]


# G6 -- sampling at a small temperature with well separated logits draws the
# argmax: the seeded run equals the argmax run token for token.
def test_g6_sampling_small_temperature_is_argmax():
    st = _setup()
    rng = RNG(3)
    tables = {}

    def lg(blk, k):
        if (blk, k) not in tables:
            t = rng.standard_normal((B, S, V))
            t[..., 7] += 10.0                # gap >> 0.1 * 19.5
            tables[(blk, k)] = t
        return tables[(blk, k)]
    a = oracle.generate(st["denoise_inputs"], lg, st["ctx_inputs"], st["kc"], st["vc"],
                        st["start"], st["end"], st["lens"], S, 2, 0.8, 0.1, MASK)
    b_ = oracle.generate(st["denoise_inputs"], lg, st["ctx_inputs"], st["kc"], st["vc"],
                         st["start"], st["end"], st["lens"], S, 2, 0.8, 0.1, MASK, seed=42)
    assert np.array_equal(a["tokens"], b_["tokens"]) and np.all(a["tokens"] == 7)
