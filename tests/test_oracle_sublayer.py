"""Pins of the oracle's weighted adaLN-single attention sublayer against facts
fixed outside it: torch's fp64 layer_norm, LayerNorm closed forms and
invariants, the separately pinned block attention reached through selection
weights, scalar-loop brute force, and permutation/gate special cases."""
import math

import numpy as np
import torch

import oracle
import oracle.sublayer as sl

RNG = np.random.default_rng


def _case(B=2, S=3, D=8, Hq=2, Hkv=1, d=4, L=(3, 0), seed=0):
    r = RNG(seed)
    T = int(sum(L)) + 1
    return dict(x=r.standard_normal((B, S, D)) * 2.0 + 0.5,
                shift=r.standard_normal((B, D)) * 0.3, scale=r.standard_normal((B, D)) * 0.3,
                gate=r.standard_normal((B, D)),
                w_qkv=r.standard_normal(((Hq + 2 * Hkv) * d, D)) / math.sqrt(D),
                w_o=r.standard_normal((D, Hq * d)) / math.sqrt(Hq * d),
                k_ctx=r.standard_normal((T, Hkv, d)), v_ctx=r.standard_normal((T, Hkv, d)),
                ctx_start=np.concatenate([[0], np.cumsum(L)[:-1]]).astype(np.int64),
                ctx_len=np.asarray(L, np.int32), n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d)


# L1 -- LayerNorm equals torch's fp64 layer_norm (no affine, eps 1e-6).
def test_l1_layer_norm_is_library_layer_norm():
    x = RNG(1).standard_normal((5, 7, 33)) * 3.0 + 1.0
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (33,), eps=1e-6).numpy()
    np.testing.assert_allclose(sl.layer_norm(x), ref, rtol=1e-12, atol=1e-12)


# L2 -- closed form at D = 2: [a, b] -> +-(a-b)/2 / sqrt((a-b)^2/4 + eps);
# L3 -- with eps = 0, rows have mean 0 and variance 1 and are invariant to
# x -> c x + t (c > 0).
def test_l2_l3_layer_norm_closed_form_and_invariants():
    for a, b in [(3.0, 1.0), (-2.0, 5.0), (0.25, 0.125)]:
        hd = (a - b) / 2.0
        s = hd / math.sqrt(hd * hd + 1e-6)
        np.testing.assert_allclose(sl.layer_norm(np.array([a, b])), [s, -s], rtol=1e-14)
    x = RNG(2).standard_normal((4, 19))
    y = sl.layer_norm(x, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y * y).mean(axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(sl.layer_norm(7.5 * x - 3.0, eps=0.0), y, rtol=1e-12, atol=1e-13)


# M1 -- modulation special cases: scale = -1 gives the shift exactly; zero
# shift and scale give LayerNorm; scale = 1 doubles it.
def test_m1_modulation_special_cases():
    c = _case(seed=3)
    x, sh = c["x"], c["shift"]
    B, S, D = x.shape
    np.testing.assert_array_equal(sl.ln_modulate(x, sh, -np.ones((B, D))), np.broadcast_to(sh[:, None, :], x.shape))
    z = np.zeros((B, D))
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (D,), eps=1e-6).numpy()
    np.testing.assert_allclose(sl.ln_modulate(x, z, z), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sl.ln_modulate(x, z, np.ones((B, D))), 2 * ref, rtol=1e-12, atol=1e-12)


# Linear -- (out, in) storage against scalar loops; q/k/v split order.
def test_linear_and_split_brute_force():
    r = RNG(4)
    x, w = r.standard_normal((2, 3, 5)), r.standard_normal((6, 5))
    y = sl.linear(x, w)
    for i in range(2):
        for j in range(3):
            for n in range(6):
                assert abs(y[i, j, n] - sum(x[i, j, k] * w[n, k] for k in range(5))) < 1e-12
    cols = np.arange(2 * 4 + 2 * 1 * 4, dtype=np.float64)[None, :]   # Hq=2, Hkv=1, d=4
    q, k, v = sl.split_qkv(cols, 2, 1, 4)
    assert q[0, 1, 0] == 4 and k[0, 0, 0] == 8 and v[0, 0, 3] == 15


# S1 -- gate = 0 or W_o = 0 leaves x exactly; inactive sequences keep x.
def test_s1_gate_and_inactive_special_cases():
    c = _case(seed=5)
    x = c["x"]
    np.testing.assert_array_equal(sl.adaln_attn_sublayer(**dict(c, gate=np.zeros_like(c["gate"]))), x)
    np.testing.assert_array_equal(sl.adaln_attn_sublayer(**dict(c, w_o=np.zeros_like(c["w_o"]))), x)
    out = sl.adaln_attn_sublayer(**c, active=np.array([0, 1], np.uint8))
    np.testing.assert_array_equal(out[0], x[0])
    np.testing.assert_allclose(out[1], sl.adaln_attn_sublayer(**c)[1], rtol=1e-13)


# S2 -- selection weights reduce the sublayer to the separately pinned block
# attention: D = Hq d, W_qkv = [I ; E_k ; E_v] (E picks channel blocks of h),
# W_o = I, so out = x + gate * block_attn(h, h_k, h_v) with h from torch's
# layer_norm.  Pins the q|k|v order, the head reshape, W_o and the gate.
def test_s2_selection_weights_reduce_to_block_attention():
    B, S, Hq, Hkv, d = 2, 3, 2, 1, 4
    D = Hq * d
    c = _case(B=B, S=S, D=D, Hq=Hq, Hkv=Hkv, d=d, seed=6)
    ek = np.zeros((Hkv * d, D))
    ev = np.zeros((Hkv * d, D))
    ek[np.arange(d), np.arange(d)] = 1.0                 # k <- channels 0..d-1 of h
    ev[np.arange(d), d + np.arange(d)] = 1.0             # v <- channels d..2d-1
    w_qkv = np.concatenate([np.eye(D), ek, ev], axis=0)
    out = sl.adaln_attn_sublayer(**dict(c, w_qkv=w_qkv, w_o=np.eye(D)))
    ln = torch.nn.functional.layer_norm(torch.from_numpy(c["x"]), (D,), eps=1e-6).numpy()
    h = ln * (1 + c["scale"][:, None, :]) + c["shift"][:, None, :]
    q = h.reshape(B, S, Hq, d)
    k = h[..., :d].reshape(B, S, Hkv, d)
    v = h[..., d:2 * d].reshape(B, S, Hkv, d)
    o, _ = oracle.block_attn(q, k, v, c["k_ctx"], c["v_ctx"], c["ctx_start"], c["ctx_len"])
    want = c["x"] + c["gate"][:, None, :] * o.reshape(B, S, D)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


# S3 -- brute force: scalar loops for LayerNorm, modulation, both
# projections, the softmax over [context ; block] and the gate.
def test_s3_brute_force_tiny():
    B, S, D, Hq, Hkv, d = 1, 2, 4, 2, 1, 2
    c = _case(B=B, S=S, D=D, Hq=Hq, Hkv=Hkv, d=d, L=(2,), seed=7)
    out = sl.adaln_attn_sublayer(**c)
    x = c["x"][0]
    h = [[0.0] * D for _ in range(S)]
    for s in range(S):
        mu = sum(x[s]) / D
        var = sum((x[s][i] - mu) ** 2 for i in range(D)) / D
        for i in range(D):
            h[s][i] = (x[s][i] - mu) / math.sqrt(var + 1e-6) * (1 + c["scale"][0][i]) + c["shift"][0][i]
    N = (Hq + 2 * Hkv) * d
    proj = [[sum(h[s][i] * c["w_qkv"][n][i] for i in range(D)) for n in range(N)] for s in range(S)]
    keys = [list(c["k_ctx"][t, 0]) for t in range(2)] + [proj[s][Hq * d:Hq * d + d] for s in range(S)]
    vals = [list(c["v_ctx"][t, 0]) for t in range(2)] + [proj[s][Hq * d + d:] for s in range(S)]
    for s in range(S):
        o = []
        for hh in range(Hq):
            qv = proj[s][hh * d:(hh + 1) * d]
            sc = [sum(qv[j] * kk[j] for j in range(d)) / math.sqrt(d) for kk in keys]
            mx = max(sc)
            e = [math.exp(v - mx) for v in sc]
            z = sum(e)
            o += [sum(e[t] * vals[t][j] for t in range(len(keys))) / z for j in range(d)]
        for n in range(D):
            y = sum(o[j] * c["w_o"][n][j] for j in range(Hq * d))
            assert abs(out[0, s, n] - (x[s][n] + c["gate"][0][n] * y)) < 1e-11


# S4 -- the block is bidirectional: permuting its slots permutes the outputs.
def test_s4_block_permutation():
    c = _case(S=5, seed=8)
    out = sl.adaln_attn_sublayer(**c)
    perm = np.array([3, 0, 4, 1, 2])
    out_p = sl.adaln_attn_sublayer(**dict(c, x=c["x"][:, perm]))
    np.testing.assert_allclose(out_p, out[:, perm], rtol=1e-12, atol=1e-12)
