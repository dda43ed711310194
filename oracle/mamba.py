"""fp64 definition of a Mamba-2 layer's sequence mixer over one block, seeded
with the context tower's boundary state (test infrastructure; see the package
header).

Pages followed (tags defined in oracle/__init__.py):
  * [dothoosh] "two-tower mechanism" section: the context tower produces
    every layer's KV cache and the final Mamba-2 states; the denoiser's
    Mamba-2 layers take their initial state directly from the context
    tower's Mamba state.
  * [modelcard] "technical features" / "implementation" notes: the seeding
    injects the context tower's conv and SSM boundary states as the initial
    states of the denoiser's Mamba layers, passed on causally (no future
    leakage); 23 of the 52 layers of each tower are Mamba-2 layers.

The Mamba-2 mixer itself is not on the pages; it is the published one (T.
Dao, A. Gu, "Transformers are SSMs", ICML 2024): a depthwise causal
convolution of width W over the channels of (x, B, C), SiLU, then per head h
with a scalar decay the selective state-space recurrence
    dt_s = softplus(dt_raw_s + dt_bias_h),   a_s = exp(dt_s * A_h),  A_h < 0
    H_s  = a_s H_{s-1} + dt_s x_s B_s^T          (H: head_dim x d_state)
    y_s  = H_s C_s + D_h x_s
with B and C shared by the heads of a group.

Readings where the pages are silent:
  * the denoiser's Mamba layers run causally over the S block slots, from the
    context's boundary state (conv state = the last W-1 pre-convolution
    inputs of the context, SSM state = H after the last context token); the
    state is read, not changed, by the denoiser (every denoising step starts
    from the same seed);
  * when a block is committed, the context tower runs the same mixer over it
    from the same seed and its final conv/SSM states become the new seed;
  * the gate (y * SiLU(z)), the norm and the projections around the mixer
    belong to the rest of the layer and are not part of this step.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def softplus(x):
    x = _f64(x)
    return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


def silu(x):
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def causal_conv(xbc, conv_state, conv_w, conv_b):
    """Depthwise causal convolution of one sequence's block with its seed.

    xbc [S, C] pre-convolution inputs, conv_state [C, W-1] (the W-1 inputs
    before the block, oldest first), conv_w [C, W], conv_b [C] ->
    SiLU(sum_j w[c, j] u[s + j] + b[c]) [S, C] where u = [conv_state^T ; xbc]
    (so w[c, W-1] multiplies the current input), and the new conv state (the
    last W-1 inputs of u).
    """
    xbc, cs, w, b = _f64(xbc), _f64(conv_state), _f64(conv_w), _f64(conv_b)
    S, C = xbc.shape
    W = w.shape[1]
    u = np.concatenate([cs.T, xbc], axis=0)                 # [W-1+S, C]
    out = np.empty((S, C))
    for s in range(S):
        out[s] = (u[s:s + W] * w.T).sum(axis=0) + b
    return silu(out), u[S:].T.copy()


def mamba_block_scan(xbc, dt_raw, conv_state, ssm_state, conv_w, conv_b, A_log, dt_bias, D,
                     n_groups, d_state, head_dim, return_state=False):
    """The Mamba-2 mixer of one layer over a block of S slots for B sequences,
    seeded with the context's conv and SSM states.

    xbc [B, S, C] with C = n_heads*head_dim + 2*n_groups*d_state, the
    channels in the order (x, B, C); dt_raw [B, S, n_heads];
    conv_state [B, C, W-1]; ssm_state [B, n_heads, head_dim, d_state];
    conv_w [C, W]; conv_b [C]; A_log, dt_bias, D [n_heads] (A = -exp(A_log)).
    Head h uses group h // (n_heads // n_groups).

    Returns y [B, S, n_heads, head_dim] (float64), and with return_state also
    the final (conv_state, ssm_state).
    """
    xbc = _f64(xbc)
    Bn, S, C = xbc.shape
    H = np.asarray(A_log).shape[0]
    P, N, G = head_dim, d_state, n_groups
    assert C == H * P + 2 * G * N and H % G == 0
    A = -np.exp(_f64(A_log))
    y = np.empty((Bn, S, H, P))
    new_conv = np.empty((Bn, C, np.asarray(conv_w).shape[1] - 1))
    new_ssm = np.empty((Bn, H, P, N))
    for b in range(Bn):
        u, new_conv[b] = causal_conv(xbc[b], conv_state[b], conv_w, conv_b)
        x = u[:, :H * P].reshape(S, H, P)
        Bm = u[:, H * P:H * P + G * N].reshape(S, G, N)
        Cm = u[:, H * P + G * N:].reshape(S, G, N)
        dt = softplus(_f64(dt_raw[b]) + _f64(dt_bias)[None, :])          # [S, H]
        for h in range(H):
            g = h // (H // G)
            st = _f64(ssm_state[b, h]).copy()
            for s in range(S):
                st = np.exp(dt[s, h] * A[h]) * st + dt[s, h] * np.outer(x[s, h], Bm[s, g])
                y[b, s, h] = st @ Cm[s, g] + _f64(D)[h] * x[s, h]
            new_ssm[b, h] = st
    if return_state:
        return y, new_conv, new_ssm
    return y


def mamba_dual_form(xbc, dt_raw, conv_state, ssm_state, conv_w, conv_b, A_log, dt_bias, D,
                    n_groups, d_state, head_dim):
    """The same outputs from the state-space duality (Dao & Gu, 2024): with
    L[s, j] = prod_{k=j+1..s} a_k (lower triangular, 1 on the diagonal),
        y_s = sum_{j<=s} L[s, j] dt_j (C_s . B_j) x_j
              + (prod_{k<=s} a_k) H_0 C_s + D x_s
    -- a quadratic, attention-like form with no recurrence.  A second,
    independent formulation used to pin mamba_block_scan."""
    xbc = _f64(xbc)
    Bn, S, C = xbc.shape
    H = np.asarray(A_log).shape[0]
    P, N, G = head_dim, d_state, n_groups
    A = -np.exp(_f64(A_log))
    y = np.empty((Bn, S, H, P))
    for b in range(Bn):
        u, _ = causal_conv(xbc[b], conv_state[b], conv_w, conv_b)
        x = u[:, :H * P].reshape(S, H, P)
        Bm = u[:, H * P:H * P + G * N].reshape(S, G, N)
        Cm = u[:, H * P + G * N:].reshape(S, G, N)
        dt = softplus(_f64(dt_raw[b]) + _f64(dt_bias)[None, :])
        for h in range(H):
            g = h // (H // G)
            la = dt[:, h] * A[h]                                   # log a_s
            cum = np.cumsum(la)
            L = np.tril(np.exp(cum[:, None] - cum[None, :]))       # prod_{j<k<=s} a_k
            M = L * (Cm[:, g] @ Bm[:, g].T) * dt[None, :, h]       # [S(s), S(j)]
            y[b, :, h] = M @ x[:, h] + np.exp(cum)[:, None] * (Cm[:, g] @ _f64(ssm_state[b, h]).T) \
                + _f64(D)[h] * x[:, h]
    return y
