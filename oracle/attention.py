"""fp64 definition of the denoiser's per-layer block attention and of the
adaLN-single timestep vectors (test infrastructure; see the package header).

Pages followed (tags defined in oracle/__init__.py):
  * [dothoosh] "two-tower mechanism" section: inside a block the denoiser
    attends bidirectionally, and causally to the earlier clean blocks; layer i
    of the denoiser talks to layer i of the context tower, whose per-layer KV
    cache covers the prompt and the committed tokens.
  * [modelcard] "technical features" section: bidirectional self-attention in
    the block plus layer-aligned cross-attention to the context tower's KV of
    the same layer; adaLN-single injects a scale, a shift and a gate per
    timestep into every denoiser layer.
  * [news] "architecture details" section: denoiser layer i cross-attends
    context-tower layer i.

Readings where the pages are silent:
  * one joint softmax over the concatenation [context keys ; block keys]
    (the block-causal mask of the dense form below);
  * scores scaled by 1/sqrt(d), no bias, no soft-cap;
  * query head h uses KV head h // (Hq / Hkv);
  * every block key is visible to every block query (masked slots included);
  * adaLN acts as q' = q * (1 + scale) + shift before the scores and
    out = residual + gate * o after them, with per-sequence vectors of width
    Hq*d broadcast over the block (parity unpinned: the pages name the three
    vectors but not where they act);
  * adaLN-single: one shared SiLU -> Linear(256 -> 3*Hq*d) plus a per-layer
    learned table, the chunks of the 3*Hq*d output taken in the order
    (shift, scale, gate); timestep embedding = the 256-wide sinusoid
    [cos(1000 t f_i), sin(1000 t f_i)], f_i = 10000^(-i/128).
"""

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def timestep_embedding(t, dim=256, max_period=10000.0, t_scale=1000.0):
    """Sinusoidal embedding of the diffusion timestep t in [0, 1].

    [dothoosh] "two-tower mechanism" and [modelcard] "technical features":
    each layer is conditioned on the diffusion timestep through adaLN-single.
    The embedding itself is not on the pages (reading: the DiT / PixArt-alpha
    sinusoid, cos half first, argument scaled by 1000).

    t: [B] -> [B, dim] float64.
    """
    t = np.asarray(t, dtype=np.float64).reshape(-1)
    half = dim // 2
    freqs = np.exp(-np.log(max_period) * np.arange(half, dtype=np.float64) / half)
    args = (t_scale * t)[:, None] * freqs[None, :]
    return np.concatenate([np.cos(args), np.sin(args)], axis=1)


def adaln_single(t_emb, w, bias, table):
    """adaLN-single: u_b = SiLU(e_b) @ W + bias, then per layer l and chunk j
    (0 = shift, 1 = scale, 2 = gate):  ada[l, j, b, :] = u_b[j*W_a:(j+1)*W_a]
    + table[l, j, :].

    [dothoosh] "two-tower mechanism": every layer is modulated by the diffusion
    timestep through adaLN-single, which adds about 1.5 M parameters;
    [modelcard] "technical features": scale, shift and gate per timestep in
    every denoiser layer.  "single" read as one shared projection plus a small
    per-layer table (PixArt-alpha's adaLN-single).

    t_emb [B, E], w [E, 3*W_a], bias [3*W_a], table [n_layers, 3, W_a]
    -> ada [n_layers, 3, B, W_a] float64.
    """
    e = _f64(t_emb)
    w = _f64(w)
    bias = _f64(bias)
    table = _f64(table)
    silu = e / (1.0 + np.exp(-e))
    u = silu @ w + bias[None, :]
    n_layers, three, width = table.shape
    assert three == 3 and u.shape[1] == 3 * width
    u = u.reshape(e.shape[0], 3, width).transpose(1, 0, 2)  # [3, B, W_a]
    return u[None, :, :, :] + table[:, :, None, :]


def modulate_q(q_blk, shift, scale):
    """q' = q * (1 + scale) + shift, per sequence b and channel (h, c), the
    vectors broadcast over the S block positions (reading of [modelcard]
    "technical features": scale and shift per timestep per layer).

    q_blk [B, S, Hq, d]; shift, scale [B, Hq*d] or None (identity).
    """
    q = _f64(q_blk)
    B, S, Hq, d = q.shape
    if scale is not None:
        q = q * (1.0 + _f64(scale).reshape(B, 1, Hq, d))
    if shift is not None:
        q = q + _f64(shift).reshape(B, 1, Hq, d)
    return q


def block_attn(q_blk, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len,
               shift=None, scale=None, gate=None, residual=None, active=None,
               return_probs=False):
    """One denoiser attention layer over [context KV of this layer ; block KV].

    For sequence b and query head h (KV head g = h // (Hq/Hkv)):
        K = [k_ctx[ctx_start[b] : ctx_start[b]+ctx_len[b], g] ; k_blk[b, :, g]]
        V likewise,  q' = modulate_q(q),  s = q' K^T / sqrt(d),
        P = softmax over keys,  o = P V,  lse = ln sum exp(s),
        out = residual + gate * o   (residual 0 and gate 1 when absent).

    [dothoosh] "two-tower mechanism" (bidirectional inside the block, causal to
    earlier clean blocks, layer i <-> layer i); [modelcard] "technical
    features" (layer-aligned cross-attention to the same layer's KV, adaLN
    scale/shift/gate).

    Shapes: q_blk [B,S,Hq,d], k_blk/v_blk [B,S,Hkv,d], k_ctx/v_ctx
    [T_ctx,Hkv,d], ctx_start [B] (token offset), ctx_len [B] (may be 0),
    shift/scale/gate [B, Hq*d], residual [B,S,Hq,d], active [B] or None.

    Returns (out [B,S,Hq,d], lse [B,S,Hq]) in float64; rows of inactive
    sequences are NaN.  With return_probs, also a dict {(b, h): P [S, L+S]}.
    """
    qm = modulate_q(q_blk, shift, scale)
    kb, vb = _f64(k_blk), _f64(v_blk)
    kc, vc = _f64(k_ctx), _f64(v_ctx)
    B, S, Hq, d = qm.shape
    Hkv = kb.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    out = np.full((B, S, Hq, d), np.nan)
    lse = np.full((B, S, Hq), np.nan)
    probs = {}
    for b in range(B):
        if active is not None and not active[b]:
            continue
        st, n = int(ctx_start[b]), int(ctx_len[b])
        for h in range(Hq):
            g = h // group
            keys = np.concatenate([kc[st:st + n, g, :], kb[b, :, g, :]], axis=0)
            vals = np.concatenate([vc[st:st + n, g, :], vb[b, :, g, :]], axis=0)
            s = qm[b, :, h, :] @ keys.T / np.sqrt(d)          # [S, n+S]
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            o = p @ vals                                       # [S, d]
            lse[b, :, h] = mx[:, 0] + np.log(z[:, 0])
            if gate is not None:
                o = o * _f64(gate)[b, h * d:(h + 1) * d][None, :]
            if residual is not None:
                o = o + _f64(residual)[b, :, h, :]
            out[b, :, h, :] = o
            if return_probs:
                probs[(b, h)] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def dense_block_causal_attn(q_seq, k_seq, v_seq, block_id):
    """Attention over one whole concatenated sequence under an explicit
    block-causal mask: position i sees position j iff block_id[j] <=
    block_id[i] (bidirectional inside a block, causal across blocks --
    [dothoosh] "two-tower mechanism").

    A second, independent formulation used to pin block_attn: the rows of the
    current block must agree with block_attn when the context is the earlier
    blocks.

    q_seq [N,Hq,d], k_seq/v_seq [N,Hkv,d], block_id [N] -> (out [N,Hq,d],
    lse [N,Hq]) float64.
    """
    q, k, v = _f64(q_seq), _f64(k_seq), _f64(v_seq)
    blk = np.asarray(block_id)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    allowed = blk[None, :] <= blk[:, None]                     # [N(i), N(j)]
    bias = np.where(allowed, 0.0, -np.inf)
    out = np.empty((N, Hq, d))
    lse = np.empty((N, Hq))
    for h in range(Hq):
        kh = k[:, h // group, :]
        vh = v[:, h // group, :]
        s = (q[:, h, :] @ kh.T) / np.sqrt(d) + bias
        mx = s.max(axis=1, keepdims=True)
        w = np.exp(s - mx)
        z = w.sum(axis=1, keepdims=True)
        out[:, h, :] = (w / z) @ vh
        lse[:, h] = mx[:, 0] + np.log(z[:, 0])
    return out, lse
