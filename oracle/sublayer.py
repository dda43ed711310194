"""fp64 definition of the denoiser's weighted adaLN-single attention sublayer
(test infrastructure; see the package header).

Pages followed (tags defined in oracle/__init__.py):
  * [dothoosh] "two-tower mechanism" section and [modelcard] "technical
    features" section: every denoiser layer is conditioned on the diffusion
    timestep through adaLN-single, which injects a scale, a shift and a gate
    per timestep into the layer; the module adds about 1.5 M parameters.
  * the attention between the projections is block_attn (this package):
    bidirectional in the block, layer-aligned to the context tower's KV.

The pages name the three vectors but not the layer around them.  Reading
(the published adaLN-single placement, PixArt-alpha / DiT, which the pages'
name refers to):
    h   = LayerNorm(x) * (1 + scale_b) + shift_b     LN without affine,
                                                     eps 1e-6, over D
    q, k, v = h W_qkv^T                              W_qkv [(Hq+2Hkv) d, D],
                                                     rows: q heads, k heads,
                                                     v heads; no bias
    o   = block_attn(q, k, v, context KV)            identity modulation
    out = x + gate_b * (o W_o^T)                     W_o [D, Hq d]; no bias
with (shift, scale, gate)_b of width D for sequence b, broadcast over the S
block slots, and no positional rotation between the projection and the
attention (the pages name none; the layer's Mamba-2 neighbours carry
position).  The pages give no hidden size D; any D works here.
"""

import numpy as np

from .attention import block_attn


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def layer_norm(x, eps=1e-6):
    """LayerNorm over the last axis without an affine map: (x - mean) /
    sqrt(var + eps), var the population variance (divide by D)."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def ln_modulate(x, shift, scale, eps=1e-6):
    """h[b, s] = LayerNorm(x[b, s]) * (1 + scale[b]) + shift[b].

    x [B, S, D]; shift, scale [B, D] -> [B, S, D] float64."""
    return layer_norm(x, eps) * (1.0 + _f64(scale)[:, None, :]) + _f64(shift)[:, None, :]


def linear(x, w):
    """x W^T for a weight stored (out_features, in_features): x [..., K],
    w [N, K] -> [..., N] float64."""
    return _f64(x) @ _f64(w).T


def split_qkv(qkv, n_q_heads, n_kv_heads, head_dim):
    """The projection's columns as q [.., Hq, d], k [.., Hkv, d], v [.., Hkv, d]."""
    qkv = _f64(qkv)
    lead = qkv.shape[:-1]
    nq, nk = n_q_heads * head_dim, n_kv_heads * head_dim
    assert qkv.shape[-1] == nq + 2 * nk
    q = qkv[..., :nq].reshape(*lead, n_q_heads, head_dim)
    k = qkv[..., nq:nq + nk].reshape(*lead, n_kv_heads, head_dim)
    v = qkv[..., nq + nk:].reshape(*lead, n_kv_heads, head_dim)
    return q, k, v


def gate_residual(x, y, gate):
    """out[b, s] = x[b, s] + gate[b] * y[b, s]; x, y [B, S, D], gate [B, D]."""
    return _f64(x) + _f64(gate)[:, None, :] * _f64(y)


def adaln_attn_sublayer(x, shift, scale, gate, w_qkv, w_o, k_ctx, v_ctx, ctx_start, ctx_len,
                        n_q_heads, n_kv_heads, head_dim, eps=1e-6, active=None,
                        return_parts=False):
    """The whole sublayer for one layer: x [B, S, D] block hidden states;
    shift, scale, gate [B, D]; w_qkv [(Hq + 2 Hkv) d, D]; w_o [D, Hq d];
    k_ctx, v_ctx [T_ctx, Hkv, d] this layer's context cache with ctx_start,
    ctx_len [B].  Inactive sequences (active[b] == 0) are left as they are
    (out = x).

    Returns out [B, S, D] float64; with return_parts also a dict of h, q,
    k, v, o (attention output [B, S, Hq, d]) and y (o W_o^T)."""
    x = _f64(x)
    B, S, D = x.shape
    h = ln_modulate(x, shift, scale, eps)
    q, k, v = split_qkv(linear(h, w_qkv), n_q_heads, n_kv_heads, head_dim)
    o, _ = block_attn(q, k, v, k_ctx, v_ctx, ctx_start, ctx_len, active=active)
    y = linear(o.reshape(B, S, n_q_heads * head_dim), w_o)
    out = gate_residual(x, y, gate)
    if active is not None:
        keep = np.asarray(active) == 0
        out[keep] = x[keep]
    if return_parts:
        return out, dict(h=h, q=q, k=k, v=v, o=o, y=y)
    return out
