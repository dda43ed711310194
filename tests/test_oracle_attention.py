"""Pins of the oracle's attention and adaLN-single against facts fixed by the
pages and by mathematics -- never against the oracle's own formula retyped.

Each test names what pins it: a library routine in a special case, an
independent formulation, a closed form, an invariant or brute force.
"""
import math

import numpy as np
import pytest
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


def _sdpa(q, k, v, mask=None):
    """torch's fp64 scaled-dot-product attention: q [H,N,d], k/v [H,M,d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask)).numpy()


# P1 -- empty context: plain bidirectional attention over the block, checked
# against torch's library attention in fp64 (GQA via repeated KV heads).
def test_p1_empty_context_is_library_attention():
    c = _case(B=2, S=6, Hq=6, Hkv=3, d=16, lens=(0, 0), seed=11)
    out, _ = oracle.block_attn(**c)
    for b in range(2):
        q = c["q_blk"][b].transpose(1, 0, 2)                    # [Hq,S,d]
        k = np.repeat(c["k_blk"][b].transpose(1, 0, 2), 2, axis=0)
        v = np.repeat(c["v_blk"][b].transpose(1, 0, 2), 2, axis=0)
        ref = _sdpa(q, k, v).transpose(1, 0, 2)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


# P2 -- equality with attention over the concatenated sequence under an explicit
# block-causal mask (independent dense formulation), with a context made of a
# prompt and two earlier committed blocks; and the dense form itself against
# torch's library attention with a boolean mask.
def test_p2_concat_block_causal_equivalence():
    S, Hq, Hkv, d = 5, 4, 2, 8
    prompt, blocks_before = 7, 2
    L = prompt + blocks_before * S
    c = _case(B=1, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(L,), seed=21)
    out, lse = oracle.block_attn(**c)
    blk_id = np.concatenate([np.zeros(prompt, int),
                             np.repeat(np.arange(1, blocks_before + 1), S),
                             np.full(S, blocks_before + 1)])
    q_ctx_rows = _rand((L, Hq, d), 99)                  # context-tower queries
    q_seq = np.concatenate([q_ctx_rows, c["q_blk"][0]], 0)
    k_seq = np.concatenate([c["k_ctx"][:L], c["k_blk"][0]], 0)
    v_seq = np.concatenate([c["v_ctx"][:L], c["v_blk"][0]], 0)
    dout, dlse = oracle.dense_block_causal_attn(q_seq, k_seq, v_seq, blk_id)
    np.testing.assert_allclose(dout[L:], out[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dlse[L:], lse[0], rtol=0, atol=1e-12)
    # the dense form against torch with the same mask
    allowed = blk_id[None, :] <= blk_id[:, None]
    ref = _sdpa(q_seq.transpose(1, 0, 2),
                np.repeat(k_seq.transpose(1, 0, 2), Hq // Hkv, 0),
                np.repeat(v_seq.transpose(1, 0, 2), Hq // Hkv, 0),
                mask=np.broadcast_to(allowed, (Hq,) + allowed.shape).copy())
    np.testing.assert_allclose(dout, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)
    # context rows are causal across blocks: the prompt must not see block 1
    assert not allowed[0, prompt]


# P3 -- probability rows sum to one and are non-negative.
def test_p3_rows_sum_to_one():
    c = _case(B=2, S=3, Hq=4, Hkv=1, d=8, lens=(9, 4), seed=31, qscale=3.0)
    _, _, probs = oracle.block_attn(**c, return_probs=True)
    for (b, h), p in probs.items():
        assert p.shape == (3, c["ctx_len"][b] + 3)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12


# P4 -- a single block slot and no context: the only key gets weight 1, so the
# output is exactly that key's value.
def test_p4_single_key_returns_value():
    c = _case(B=3, S=1, Hq=4, Hkv=2, d=8, lens=(0, 0, 0), seed=41)
    out, lse = oracle.block_attn(**c)
    for b in range(3):
        for h in range(4):
            np.testing.assert_array_equal(out[b, 0, h], c["v_blk"][b, 0, h // 2])
    # lse of a single key is its score
    s = (c["q_blk"][0, 0, 0] @ c["k_blk"][0, 0, 0]) / math.sqrt(8)
    assert abs(lse[0, 0, 0] - s) < 1e-12


# P5 -- all keys equal: uniform weights, output = mean of the values,
# lse = score + ln(number of keys).
def test_p5_equal_keys_give_mean_value():
    c = _case(B=1, S=3, Hq=2, Hkv=1, d=4, lens=(6,), seed=51)
    key = _rand((4,), 52)
    c["k_ctx"][:] = key
    c["k_blk"][:] = key
    out, lse = oracle.block_attn(**c)
    vals = np.concatenate([c["v_ctx"][:6, 0], c["v_blk"][0, :, 0]], 0)
    for s in range(3):
        for h in range(2):
            np.testing.assert_allclose(out[0, s, h], vals.mean(0), atol=1e-13)
            score = c["q_blk"][0, s, h] @ key / 2.0
            assert abs(lse[0, s, h] - (score + math.log(9))) < 1e-12


# P6 -- one planted key whose score exceeds n-1 equal others by delta gets
# weight e^delta / (e^delta + n - 1).
@pytest.mark.parametrize("delta", [0.5, 3.0, 9.0])
def test_p6_planted_key_weight(delta):
    d, L, S = 8, 10, 2
    c = _case(B=1, S=S, Hq=1, Hkv=1, d=d, lens=(L,), seed=61)
    q = np.zeros(d)
    q[0] = 1.0
    c["q_blk"][0, :, 0] = q
    c["k_ctx"][:, 0] = 0.0
    c["k_blk"][0, :, 0] = 0.0
    c["k_ctx"][3, 0, 0] = delta * math.sqrt(d)           # planted at ctx slot 3
    vals = np.zeros((L + S, d))
    c["v_ctx"][:L, 0] = 0.0
    c["v_blk"][0, :, 0] = 0.0
    c["v_ctx"][3, 0, 1] = 1.0
    vals[3, 1] = 1.0
    n = L + S
    expect = math.exp(delta) / (math.exp(delta) + n - 1)
    out, _, probs = oracle.block_attn(**c, return_probs=True)
    assert abs(probs[(0, 0)][0, 3] - expect) < 1e-14
    assert abs(out[0, 0, 0, 1] - expect) < 1e-14


# P7 -- adaLN special cases: identity vectors change nothing; gate 0 returns the
# residual; scale = -1 with shift 0 zeroes the query (uniform weights over all
# L+S keys, lse = ln(L+S)); gate 2 doubles the attention term.
def test_p7_adaln_special_cases():
    B, S, Hq, Hkv, d = 2, 4, 4, 2, 8
    c = _case(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(7, 3), seed=71)
    W = Hq * d
    plain, plain_lse = oracle.block_attn(**c)
    ident, ident_lse = oracle.block_attn(**c, shift=np.zeros((B, W)),
                                         scale=np.zeros((B, W)), gate=np.ones((B, W)))
    np.testing.assert_array_equal(plain, ident)
    np.testing.assert_array_equal(plain_lse, ident_lse)
    res = _rand((B, S, Hq, d), 72)
    zero_gate, _ = oracle.block_attn(**c, gate=np.zeros((B, W)), residual=res)
    np.testing.assert_array_equal(zero_gate, res)
    two, _ = oracle.block_attn(**c, gate=np.full((B, W), 2.0), residual=res)
    np.testing.assert_allclose(two, res + 2 * plain, atol=1e-13)
    flat, flat_lse = oracle.block_attn(**c, scale=np.full((B, W), -1.0),
                                       shift=np.zeros((B, W)))
    for b in range(B):
        L = int(c["ctx_len"][b])
        st = int(c["ctx_start"][b])
        for h in range(Hq):
            vals = np.concatenate([c["v_ctx"][st:st + L, h // 2], c["v_blk"][b, :, h // 2]], 0)
            np.testing.assert_allclose(flat[b, :, h], np.broadcast_to(vals.mean(0), (S, d)),
                                       atol=1e-13)
            np.testing.assert_allclose(flat_lse[b, :, h], math.log(L + S), atol=1e-13)
    # a shift alone moves the query: shift = -q cancels it (scale 0)
    qflat = c["q_blk"].reshape(B, S, W)
    if S > 1:
        # per-sequence shift can cancel only one slot; cancel slot 0
        cancel, cancel_lse = oracle.block_attn(**c, shift=-qflat[:, 0, :],
                                               scale=np.zeros((B, W)))
        np.testing.assert_allclose(cancel[:, 0], flat[:, 0], atol=1e-13)


# P8 -- permutation invariances: permuting the block slots jointly in (q, k, v)
# permutes the outputs; permuting the context tokens changes nothing; moving a
# sequence's context elsewhere in the cache changes nothing.
def test_p8_permutations():
    c = _case(B=2, S=5, Hq=4, Hkv=2, d=8, lens=(6, 9), seed=81)
    out, lse = oracle.block_attn(**c)
    perm = RNG(82).permutation(5)
    c2 = dict(c)
    c2["q_blk"] = c["q_blk"][:, perm]
    c2["k_blk"] = c["k_blk"][:, perm]
    c2["v_blk"] = c["v_blk"][:, perm]
    out2, lse2 = oracle.block_attn(**c2)
    np.testing.assert_allclose(out2, out[:, perm], atol=1e-12)
    np.testing.assert_allclose(lse2, lse[:, perm], atol=1e-12)
    c3 = dict(c)
    kc, vc = c["k_ctx"].copy(), c["v_ctx"].copy()
    for b in range(2):
        st, n = int(c["ctx_start"][b]), int(c["ctx_len"][b])
        p = RNG(83 + b).permutation(n)
        kc[st:st + n] = c["k_ctx"][st:st + n][p]
        vc[st:st + n] = c["v_ctx"][st:st + n][p]
    c3["k_ctx"], c3["v_ctx"] = kc, vc
    out3, _ = oracle.block_attn(**c3)
    np.testing.assert_allclose(out3, out, atol=1e-12)
    # relocate: sequence 1 first, then a gap, then sequence 0
    c4 = dict(c)
    n0, n1 = int(c["ctx_len"][0]), int(c["ctx_len"][1])
    gap = 3
    kc4 = np.zeros((n1 + gap + n0,) + c["k_ctx"].shape[1:])
    vc4 = np.zeros_like(kc4)
    kc4[:n1] = c["k_ctx"][n0:n0 + n1]
    vc4[:n1] = c["v_ctx"][n0:n0 + n1]
    kc4[n1 + gap:] = c["k_ctx"][:n0]
    vc4[n1 + gap:] = c["v_ctx"][:n0]
    c4["k_ctx"], c4["v_ctx"] = kc4, vc4
    c4["ctx_start"] = np.array([n1 + gap, 0], np.int64)
    out4, _ = oracle.block_attn(**c4)
    np.testing.assert_allclose(out4, out, atol=1e-12)


# P9 -- GQA equals MHA with each KV head repeated for its query group
# (contiguous groups: query head h reads KV head h // (Hq/Hkv)).
def test_p9_gqa_is_repeated_mha():
    c = _case(B=2, S=3, Hq=6, Hkv=2, d=8, lens=(4, 5), seed=91)
    out, lse = oracle.block_attn(**c)
    m = dict(c)
    for key in ("k_blk", "v_blk", "k_ctx", "v_ctx"):
        ax = 2 if key.endswith("blk") else 1
        m[key] = np.repeat(c[key], 3, axis=ax)
    out2, lse2 = oracle.block_attn(**m)
    np.testing.assert_allclose(out2, out, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    # a head-mapping mistake (h % Hkv) would differ: heads 1 and 3 use different KV
    assert not np.allclose(out[:, :, 1], out[:, :, 3])


# Brute force -- scalar loops with math.exp on tiny shapes, every optional
# input present, inactive sequence included.
def _brute(c, shift, scale, gate, res, active):
    B, S, Hq, d = c["q_blk"].shape
    Hkv = c["k_blk"].shape[2]
    out = np.full((B, S, Hq, d), np.nan)
    lse = np.full((B, S, Hq), np.nan)
    for b in range(B):
        if not active[b]:
            continue
        st, n = int(c["ctx_start"][b]), int(c["ctx_len"][b])
        for s in range(S):
            for h in range(Hq):
                g = h * Hkv // Hq
                qv = [c["q_blk"][b, s, h, i] * (1 + scale[b, h * d + i]) + shift[b, h * d + i]
                      for i in range(d)]
                keys = [c["k_ctx"][st + t, g] for t in range(n)] + [c["k_blk"][b, t, g] for t in range(S)]
                vals = [c["v_ctx"][st + t, g] for t in range(n)] + [c["v_blk"][b, t, g] for t in range(S)]
                sc = [sum(qv[i] * kk[i] for i in range(d)) / math.sqrt(d) for kk in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                z = sum(w)
                lse[b, s, h] = mx + math.log(z)
                for i in range(d):
                    o = sum(w[t] * vals[t][i] for t in range(len(w))) / z
                    out[b, s, h, i] = res[b, s, h, i] + gate[b, h * d + i] * o
    return out, lse


def test_brute_force_tiny():
    B, S, Hq, Hkv, d = 3, 3, 4, 2, 4
    c = _case(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, lens=(5, 0, 2), seed=101)
    W = Hq * d
    shift, scale, gate = _rand((B, W), 102, .3), _rand((B, W), 103, .3), _rand((B, W), 104)
    res = _rand((B, S, Hq, d), 105)
    active = np.array([1, 1, 0], np.uint8)
    out, lse = oracle.block_attn(**c, shift=shift, scale=scale, gate=gate,
                                 residual=res, active=active)
    bout, blse = _brute(c, shift, scale, gate, res, active)
    np.testing.assert_allclose(out[:2], bout[:2], atol=1e-12)
    np.testing.assert_allclose(lse[:2], blse[:2], atol=1e-12)
    assert np.isnan(out[2]).all() and np.isnan(lse[2]).all()


# adaLN-single pins: sinusoid special values; SiLU against torch's library SiLU;
# e = 0 gives bias + table (SiLU(0) = 0); scalar-loop brute force of the map.
def test_timestep_embedding_special_values():
    e = oracle.timestep_embedding([0.0, 0.25, 1.0])
    assert e.shape == (3, 256)
    np.testing.assert_array_equal(e[0, :128], 1.0)
    np.testing.assert_array_equal(e[0, 128:], 0.0)
    # frequency 0 is 1 (argument 1000 t); frequency 64 is 10000^-0.5 = 0.01
    for i, t in enumerate([0.0, 0.25, 1.0]):
        assert abs(e[i, 0] - math.cos(1000 * t)) < 1e-15
        assert abs(e[i, 128] - math.sin(1000 * t)) < 1e-15
        assert abs(e[i, 64] - math.cos(10 * t)) < 1e-13
        assert abs(e[i, 192] - math.sin(10 * t)) < 1e-13
    # each (cos, sin) pair lies on the unit circle
    np.testing.assert_allclose(e[:, :128] ** 2 + e[:, 128:] ** 2, 1.0, atol=1e-14)


# Structure of the sinusoid, checked without its formula: the angle-addition
# identities hold for every pair (so each pair is (cos, sin) of one angle that
# is linear in t), and the angular frequencies recovered from the phase at a
# small t form one geometric progression from 1000 down by a factor of
# 10000 per 128 pairs (max period 10000, argument scale 1000).
def test_timestep_embedding_angle_addition_and_frequencies():
    rng = np.random.default_rng(7)
    t1, t2 = rng.uniform(0, 0.5, 16), rng.uniform(0, 0.5, 16)
    a, b, ab = (oracle.timestep_embedding(t1), oracle.timestep_embedding(t2),
                oracle.timestep_embedding(t1 + t2))
    ca, sa, cb, sb = a[:, :128], a[:, 128:], b[:, :128], b[:, 128:]
    np.testing.assert_allclose(ab[:, :128], ca * cb - sa * sb, atol=1e-12)
    np.testing.assert_allclose(ab[:, 128:], sa * cb + ca * sb, atol=1e-12)
    t = 1e-6   # every phase 1000 t f_i stays below pi
    e = oracle.timestep_embedding([t])[0]
    omega = np.arctan2(e[128:], e[:128]) / t
    assert abs(omega[0] - 1000.0) < 1e-6
    ratio = omega[1:] / omega[:-1]
    np.testing.assert_allclose(ratio, 10000.0 ** (-1.0 / 128), rtol=1e-9)
    assert abs(omega[-1] / omega[0] - 10000.0 ** (-127.0 / 128)) < 1e-9


def test_adaln_single_pins():
    B, E, width, nl = 3, 6, 4, 2
    emb = _rand((B, E), 111, 2.0)
    w = _rand((E, 3 * width), 112)
    bias = _rand((3 * width,), 113)
    table = _rand((nl, 3, width), 114)
    ada = oracle.adaln_single(emb, w, bias, table)
    assert ada.shape == (nl, 3, B, width)
    # e = 0 -> SiLU(0) = 0 -> ada = bias chunk + table
    z = oracle.adaln_single(np.zeros((B, E)), w, bias, table)
    for l in range(nl):
        for j in range(3):
            np.testing.assert_array_equal(z[l, j], np.broadcast_to(bias[j * width:(j + 1) * width] + table[l, j], (B, width)))
    # identity weight, zero bias and table: the shift chunk is SiLU(e) itself
    ident = oracle.adaln_single(emb[:, :width], np.eye(width, 3 * width), np.zeros(3 * width),
                                np.zeros((1, 3, width)))
    ref = torch.nn.functional.silu(torch.from_numpy(emb[:, :width])).numpy()
    np.testing.assert_allclose(ident[0, 0], ref, atol=1e-15)
    np.testing.assert_array_equal(ident[0, 1], 0.0)
    # scalar-loop brute force
    for l in range(nl):
        for j in range(3):
            for b in range(B):
                for c in range(width):
                    col = j * width + c
                    u = sum((emb[b, k] / (1 + math.exp(-emb[b, k]))) * w[k, col] for k in range(E))
                    assert abs(ada[l, j, b, c] - (u + bias[col] + table[l, j, c])) < 1e-12
