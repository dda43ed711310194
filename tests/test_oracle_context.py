"""Pins of the oracle's context-tower step (causal attention over a committed
block, cache append, length rule) against facts fixed by the pages and by
mathematics -- never against the oracle's own formula retyped.

Each test names what pins it: a library routine in a special case, an
independent formulation, an equivalence with the (separately pinned)
denoiser attention, an invariant or brute force.
"""
import math

import numpy as np
import torch

import oracle

RNG = np.random.default_rng


def _rand(shape, seed, scale=1.0):
    return RNG(seed).standard_normal(shape) * scale


def _case(B=2, S=4, Hq=4, Hkv=2, d=8, lens=(5, 0), seed=0, qscale=1.0):
    lens = list(lens)[:B]
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return dict(
        q_blk=_rand((B, S, Hq, d), seed, qscale),
        k_blk=_rand((B, S, Hkv, d), seed + 1),
        v_blk=_rand((B, S, Hkv, d), seed + 2),
        k_ctx=_rand((max(total, 1), Hkv, d), seed + 3),
        v_ctx=_rand((max(total, 1), Hkv, d), seed + 4),
        ctx_start=starts,
        ctx_len=np.asarray(lens, dtype=np.int32),
    )


# C1 -- empty context: textbook causal self-attention over the block, checked
# against torch's fp64 scaled-dot-product attention with is_causal=True (GQA
# through repeated KV heads).
def test_c1_empty_context_is_library_causal_attention():
    c = _case(B=2, S=7, Hq=6, Hkv=3, d=16, lens=(0, 0), seed=21)
    out, lse = oracle.ctx_block_attn(**c)
    for b in range(2):
        q = torch.from_numpy(c["q_blk"][b].transpose(1, 0, 2).copy())
        k = torch.from_numpy(np.repeat(c["k_blk"][b].transpose(1, 0, 2), 2, axis=0).copy())
        v = torch.from_numpy(np.repeat(c["v_blk"][b].transpose(1, 0, 2), 2, axis=0).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        np.testing.assert_allclose(out[b], ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
        s = (q @ k.transpose(1, 2)) / math.sqrt(16)
        s = s.masked_fill(torch.triu(torch.ones(7, 7, dtype=torch.bool), 1), float("-inf"))
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy().T, rtol=0, atol=1e-12)


# C2 -- independent dense formulation: the concatenated sequence [context ;
# block] under the block-causal mask with every new token in a block of its
# own is token-causal attention; its block rows must equal ctx_block_attn.
# (The dense routine is itself pinned against torch's masked attention.)
def test_c2_dense_mask_with_one_block_per_token():
    B, S, Hq, Hkv, d = 2, 5, 4, 2, 8
    c = _case(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(9, 3), seed=22)
    out, lse = oracle.ctx_block_attn(**c)
    for b in range(B):
        st, n = int(c["ctx_start"][b]), int(c["ctx_len"][b])
        q_seq = np.concatenate([_rand((n, Hq, d), 99 + b), c["q_blk"][b]], axis=0)
        k_seq = np.concatenate([c["k_ctx"][st:st + n], c["k_blk"][b]], axis=0)
        v_seq = np.concatenate([c["v_ctx"][st:st + n], c["v_blk"][b]], axis=0)
        blk = np.concatenate([np.zeros(n, dtype=int), np.arange(1, S + 1)])
        ro, rl = oracle.dense_block_causal_attn(q_seq, k_seq, v_seq, blk)
        np.testing.assert_allclose(out[b], ro[n:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl[n:], rtol=0, atol=1e-12)


# C3 -- autoregressive equivalence: block token s is what a one-token decode
# step computes when the context already holds block tokens 0..s-1 -- the
# denoiser's attention (pinned separately) with S = 1 over [context ; block
# tokens < s] and the token's own key as the single block key.
def test_c3_row_equals_single_token_decode():
    B, S, Hq, Hkv, d = 2, 6, 8, 2, 16
    c = _case(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(11, 0), seed=23)
    out, lse = oracle.ctx_block_attn(**c)
    for b in range(B):
        st, n = int(c["ctx_start"][b]), int(c["ctx_len"][b])
        for s in range(S):
            kc = np.concatenate([c["k_ctx"][st:st + n], c["k_blk"][b, :s]], axis=0)
            vc = np.concatenate([c["v_ctx"][st:st + n], c["v_blk"][b, :s]], axis=0)
            o1, l1 = oracle.block_attn(c["q_blk"][b:b + 1, s:s + 1], c["k_blk"][b:b + 1, s:s + 1],
                                       c["v_blk"][b:b + 1, s:s + 1], kc, vc, np.array([0]),
                                       np.array([n + s]))
            np.testing.assert_allclose(out[b, s], o1[0, 0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, s], l1[0, 0], rtol=0, atol=1e-12)


# C4 -- special cases: the last block token sees every key, exactly like the
# denoiser's bidirectional attention; with no context the first token sees
# only itself, so its output is its value row exactly.
def test_c4_last_row_bidirectional_first_row_value():
    c = _case(B=2, S=5, Hq=4, Hkv=1, d=8, lens=(6, 0), seed=24)
    out, lse = oracle.ctx_block_attn(**c)
    bo, bl = oracle.block_attn(**c)
    np.testing.assert_allclose(out[:, -1], bo[:, -1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, -1], bl[:, -1], rtol=0, atol=1e-12)
    for h in range(4):
        np.testing.assert_array_equal(out[1, 0, h], c["v_blk"][1, 0, 0])
        s0 = c["q_blk"][1, 0, h] @ c["k_blk"][1, 0, 0] / math.sqrt(8)
        assert abs(lse[1, 0, h] - s0) < 1e-12


# C5 -- causality: changing the keys and values of block tokens after s
# leaves row s unchanged (and does change the rows that see them); permuting
# context tokens changes nothing (a set of keys, no positions).
def test_c5_causality_and_context_permutation():
    c = _case(B=1, S=6, Hq=4, Hkv=2, d=8, lens=(7,), seed=25)
    out, _ = oracle.ctx_block_attn(**c)
    for s in range(5):
        c2 = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v) for k, v in c.items()}
        c2["k_blk"][0, s + 1:] += 3.0
        c2["v_blk"][0, s + 1:] -= 2.0
        out2, _ = oracle.ctx_block_attn(**c2)
        np.testing.assert_array_equal(out2[0, :s + 1], out[0, :s + 1])
        assert np.abs(out2[0, s + 1:] - out[0, s + 1:]).min() > 0
    perm = RNG(5).permutation(7)
    c3 = dict(c, k_ctx=c["k_ctx"][perm], v_ctx=c["v_ctx"][perm])
    out3, _ = oracle.ctx_block_attn(**c3)
    np.testing.assert_allclose(out3, out, rtol=0, atol=1e-12)


# C6 -- brute force: scalar loops over every (b, h, s) and visible key, with
# the residual and an inactive sequence.
def test_c6_brute_force_tiny():
    B, S, Hq, Hkv, d = 3, 3, 4, 2, 4
    c = _case(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(2, 0, 4), seed=26)
    res = _rand((B, S, Hq, d), 27)
    active = np.array([1, 1, 0], dtype=np.uint8)
    out, lse = oracle.ctx_block_attn(**c, residual=res, active=active)
    for b in range(B):
        if not active[b]:
            assert np.isnan(out[b]).all() and np.isnan(lse[b]).all()
            continue
        st, n = int(c["ctx_start"][b]), int(c["ctx_len"][b])
        for h in range(Hq):
            g = h * Hkv // Hq
            for s in range(S):
                ks = [c["k_ctx"][st + j, g] for j in range(n)] + [c["k_blk"][b, j, g] for j in range(s + 1)]
                vs = [c["v_ctx"][st + j, g] for j in range(n)] + [c["v_blk"][b, j, g] for j in range(s + 1)]
                sc = []
                for kk in ks:
                    acc = 0.0
                    for i in range(d):
                        acc += c["q_blk"][b, s, h, i] * kk[i]
                    sc.append(acc / math.sqrt(d))
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                for i in range(d):
                    o = math.fsum(w[j] * vs[j][i] for j in range(len(w))) / z
                    assert abs(out[b, s, h, i] - (o + res[b, s, h, i])) < 1e-12
                assert abs(lse[b, s, h] - (m + math.log(z))) < 1e-12


# K1 -- cache append on hand-built regions: sequence 0 has room, sequence 1
# is exactly full after the append, sequence 2 has no room, sequence 3 is
# inactive.  Only the appended rows change, the block lands right after the
# context, and the length rule uses the same room test.
def test_k1_append_regions_and_length_rule():
    Hkv, d, S = 2, 4, 3
    starts = np.array([0, 10, 20, 30], dtype=np.int64)
    ends = np.array([10, 17, 24, 40], dtype=np.int64)
    lens = np.array([2, 4, 2, 1], dtype=np.int32)
    active = np.array([1, 1, 1, 0], dtype=np.uint8)
    kc = np.arange(40 * Hkv * d, dtype=np.float64).reshape(40, Hkv, d)
    vc = -kc
    kb = 1000.0 + np.arange(4 * S * Hkv * d, dtype=np.float64).reshape(4, S, Hkv, d)
    vb = -kb
    nk, nv, app = oracle.kv_append(kc, vc, kb, vb, starts, ends, lens, active)
    assert app.tolist() == [True, True, False, False]
    expect_k = kc.copy()
    expect_k[2:5] = kb[0]
    expect_k[14:17] = kb[1]
    np.testing.assert_array_equal(nk, expect_k)
    np.testing.assert_array_equal(nv, -expect_k)
    assert (kc == np.arange(40 * Hkv * d).reshape(40, Hkv, d)).all()   # input untouched
    n2, app2 = oracle.ctx_advance(S, starts, ends, lens, active)
    assert n2.tolist() == [5, 7, 2, 1]
    assert app2.tolist() == app.tolist()


# K2 -- the append plus the length rule turn the next layer call into plain
# attention over the grown context: after appending block A, the denoiser's
# attention for block B over the grown cache equals attention over the
# explicit concatenation [context ; A] (state carried across blocks).
def test_k2_grown_context_feeds_next_block():
    B, S, Hq, Hkv, d = 2, 4, 4, 2, 8
    c = _case(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(5, 0), seed=28)
    cap = 5 + 2 * S
    starts = np.array([0, cap], dtype=np.int64)
    ends = starts + cap
    kc = np.zeros((2 * cap, Hkv, d))
    vc = np.zeros((2 * cap, Hkv, d))
    kc[0:5], vc[0:5] = c["k_ctx"][0:5], c["v_ctx"][0:5]
    nk, nv, app = oracle.kv_append(kc, vc, c["k_blk"], c["v_blk"], starts, ends, c["ctx_len"])
    n2, _ = oracle.ctx_advance(S, starts, ends, c["ctx_len"])
    assert app.all() and n2.tolist() == [5 + S, S]
    q2 = _rand((B, S, Hq, d), 29)
    k2, v2 = _rand((B, S, Hkv, d), 30), _rand((B, S, Hkv, d), 31)
    out, _ = oracle.block_attn(q2, k2, v2, nk, nv, starts, n2)
    for b in range(B):
        st = int(c["ctx_start"][b])
        n = int(c["ctx_len"][b])
        kcat = np.concatenate([c["k_ctx"][st:st + n], c["k_blk"][b]], axis=0)
        vcat = np.concatenate([c["v_ctx"][st:st + n], c["v_blk"][b]], axis=0)
        ref, _ = oracle.block_attn(q2[b:b + 1], k2[b:b + 1], v2[b:b + 1], kcat, vcat,
                                   np.array([0]), np.array([n + S]))
        np.testing.assert_allclose(out[b], ref[0], rtol=0, atol=1e-12)
