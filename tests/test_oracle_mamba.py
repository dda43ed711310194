"""Pins of the oracle's seeded Mamba-2 block scan against facts fixed by the
mathematics -- never against the oracle's own recurrence retyped: the
state-space duality's quadratic form, the seeding composition property,
numpy's convolution, closed forms and brute force."""
import math

import numpy as np

import oracle.mamba as mb

RNG = np.random.default_rng


def _case(B=2, S=5, H=4, P=3, N=4, G=2, W=4, seed=0, dt_shift=0.0):
    r = RNG(seed)
    C = H * P + 2 * G * N
    return dict(xbc=r.standard_normal((B, S, C)), dt_raw=r.standard_normal((B, S, H)) + dt_shift,
                conv_state=r.standard_normal((B, C, W - 1)),
                ssm_state=r.standard_normal((B, H, P, N)),
                conv_w=r.standard_normal((C, W)) * 0.5, conv_b=r.standard_normal(C) * 0.1,
                A_log=r.standard_normal(H) * 0.5, dt_bias=r.standard_normal(H) * 0.3,
                D=r.standard_normal(H), n_groups=G, d_state=N, head_dim=P)


# M1 -- the recurrence equals the state-space duality's quadratic form
# (Dao & Gu, 2024): y = (L o C B^T dt) x + decay * H0 C + D x.
def test_m1_scan_equals_dual_form():
    for seed in range(3):
        c = _case(seed=seed, S=7)
        np.testing.assert_allclose(mb.mamba_block_scan(**c), mb.mamba_dual_form(**c),
                                   rtol=1e-12, atol=1e-12)


# M2 -- seeding composition: the context scanned from zero states, then the
# block scanned from the context's final states, gives the block outputs of
# one scan over [context ; block] from zero states (causal: no leakage).
def test_m2_seeded_block_equals_scan_of_concatenation():
    c = _case(S=9, seed=4)
    B, S, C = c["xbc"].shape
    H, P, N = 4, 3, 4
    zero_conv = np.zeros_like(c["conv_state"])
    zero_ssm = np.zeros_like(c["ssm_state"])
    full = dict(c, conv_state=zero_conv, ssm_state=zero_ssm)
    y_full = mb.mamba_block_scan(**full)
    Lc = 6                                       # context = first 6 tokens
    ctx = dict(full, xbc=c["xbc"][:, :Lc], dt_raw=c["dt_raw"][:, :Lc])
    _, conv1, ssm1 = mb.mamba_block_scan(**ctx, return_state=True)
    blk = dict(c, xbc=c["xbc"][:, Lc:], dt_raw=c["dt_raw"][:, Lc:], conv_state=conv1,
               ssm_state=ssm1)
    np.testing.assert_allclose(mb.mamba_block_scan(**blk), y_full[:, Lc:], rtol=1e-12,
                               atol=1e-12)
    # the new conv state is the last W-1 raw inputs of the context
    np.testing.assert_array_equal(conv1, np.transpose(c["xbc"][:, Lc - 3:Lc], (0, 2, 1)))
    assert y_full.shape == (B, S, H, P)


# M3 -- the causal depthwise convolution against numpy.convolve per channel
# over [seed ; block] (numpy flips the kernel, so the tap order is pinned).
def test_m3_conv_against_numpy():
    r = RNG(5)
    S, C, W = 6, 5, 4
    xbc, cs = r.standard_normal((S, C)), r.standard_normal((C, W - 1))
    w, b = r.standard_normal((C, W)), r.standard_normal(C)
    out, new_state = mb.causal_conv(xbc, cs, w, b)
    for ch in range(C):
        u = np.concatenate([cs[ch], xbc[:, ch]])
        ref = np.convolve(u, w[ch][::-1], mode="valid") + b[ch]
        np.testing.assert_allclose(out[:, ch], ref / (1 + np.exp(-ref)), rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(new_state, xbc[-3:].T)


# M4 -- closed forms: an instant decay (A -> -inf) leaves no memory,
# y_s = dt_s (C_s . B_s) x_s + D x_s; a zero step (dt -> 0) keeps the seed,
# y_s = H0 C_s + D x_s and the final state is the seed.
def test_m4_closed_forms():
    c = _case(S=4, seed=6)
    H, P, N, G = 4, 3, 4, 2
    fast = dict(c, A_log=np.full(H, 8.0))              # A = -e^8: a = exp(-2981 dt) = 0
    y = mb.mamba_block_scan(**fast)
    for b in range(2):
        u, _ = mb.causal_conv(c["xbc"][b], c["conv_state"][b], c["conv_w"], c["conv_b"])
        x = u[:, :H * P].reshape(4, H, P)
        Bm = u[:, H * P:H * P + G * N].reshape(4, G, N)
        Cm = u[:, H * P + G * N:].reshape(4, G, N)
        dt = mb.softplus(c["dt_raw"][b] + c["dt_bias"])
        for h in range(H):
            g = h // 2
            for s in range(4):
                want = dt[s, h] * (Cm[s, g] @ Bm[s, g]) * x[s, h] + c["D"][h] * x[s, h]
                np.testing.assert_allclose(y[b, s, h], want, rtol=1e-12, atol=1e-12)
    still = dict(c, dt_raw=np.full_like(c["dt_raw"], -800.0), dt_bias=np.zeros(H))
    y2, _, ssm = mb.mamba_block_scan(**still, return_state=True)
    np.testing.assert_array_equal(ssm, c["ssm_state"])
    for b in range(2):
        u, _ = mb.causal_conv(c["xbc"][b], c["conv_state"][b], c["conv_w"], c["conv_b"])
        x = u[:, :H * P].reshape(4, H, P)
        Cm = u[:, H * P + G * N:].reshape(4, G, N)
        for h in range(H):
            want = Cm[:, h // 2] @ c["ssm_state"][b, h].T + c["D"][h] * x[:, h]
            np.testing.assert_allclose(y2[b, :, h], want, rtol=1e-12, atol=1e-12)


# M5 -- brute force: scalar loops over every (b, h, s, p, n), with its own
# convolution, softplus and group map.
def test_m5_brute_force_tiny():
    c = _case(B=1, S=3, H=4, P=2, N=3, G=2, W=3, seed=7)
    y = mb.mamba_block_scan(**c)
    H, P, N, G, W, S = 4, 2, 3, 2, 3, 3
    C = H * P + 2 * G * N
    conv = [[0.0] * C for _ in range(S)]
    for s in range(S):
        for ch in range(C):
            acc = c["conv_b"][ch]
            for j in range(W):
                t = s + j - (W - 1)
                v = c["conv_state"][0, ch, W - 1 + t] if t < 0 else c["xbc"][0, t, ch]
                acc += c["conv_w"][ch, j] * v
            conv[s][ch] = acc / (1.0 + math.exp(-acc))
    for h in range(H):
        g = h // (H // G)
        A = -math.exp(c["A_log"][h])
        st = [[c["ssm_state"][0, h, p, n] for n in range(N)] for p in range(P)]
        for s in range(S):
            z = c["dt_raw"][0, s, h] + c["dt_bias"][h]
            dt = math.log1p(math.exp(z))
            a = math.exp(dt * A)
            for p in range(P):
                xv = conv[s][h * P + p]
                out = 0.0
                for n in range(N):
                    bv = conv[s][H * P + g * N + n]
                    cv = conv[s][H * P + G * N + g * N + n]
                    st[p][n] = a * st[p][n] + dt * xv * bv
                    out += st[p][n] * cv
                assert abs(y[0, s, h, p] - (out + c["D"][h] * xv)) < 1e-12


# M6 -- causality inside the block: changing the inputs of later slots
# leaves earlier outputs unchanged (and changes the later ones).
def test_m6_causal_in_block():
    c = _case(S=6, seed=8)
    y = mb.mamba_block_scan(**c)
    for s in range(5):
        c2 = dict(c, xbc=c["xbc"].copy(), dt_raw=c["dt_raw"].copy())
        c2["xbc"][:, s + 1:] += 1.0
        c2["dt_raw"][:, s + 1:] -= 0.5
        y2 = mb.mamba_block_scan(**c2)
        np.testing.assert_array_equal(y2[:, :s + 1], y[:, :s + 1])
        assert np.abs(y2[:, s + 1:] - y[:, s + 1:]).max() > 0
