"""fp64 definition of the context tower's step over a committed block
(test infrastructure; see the package header).

Pages followed (tags defined in oracle/__init__.py):
  * [dothoosh] "two-tower mechanism" section: the frozen context tower runs
    causally over the prompt and the committed tokens and produces every
    layer's KV cache (and the final Mamba-2 states); the denoiser reads that
    cache layer by layer.
  * [news] "architecture details" section: the autoregressive context tower
    keeps the backbone's AR behaviour and is the part that generates the KV
    cache.

Readings where the pages are silent:
  * once a block is final, the context tower consumes its S tokens like an
    autoregressive prefill chunk: block token s sees every context token of
    its sequence and the block tokens 0..s (causal inside the block), one
    softmax over all visible keys, scores scaled by 1/sqrt(d), query head h
    on KV head h // (Hq / Hkv), no adaLN (the timestep modulation belongs to
    the denoiser only);
  * the block's per-layer K/V are then appended to that layer's cache right
    after the sequence's context, and the context length grows by S; a
    sequence whose reserved cache region [ctx_start, ctx_end) has no room for
    S more tokens is left untouched and reported as not appended.
"""

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def ctx_block_attn(q_blk, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, residual=None,
                   active=None):
    """The context tower's attention for the S tokens of a committed block.

    For sequence b, query head h (KV head g = h // (Hq/Hkv)) and block token s:
        K_s = [k_ctx[ctx_start[b] : ctx_start[b]+ctx_len[b], g] ; k_blk[b, 0..s, g]]
        V_s likewise,  scores = q[b, s, h] K_s^T / sqrt(d),
        o = softmax(scores) V_s,  lse = ln sum exp(scores),
        out = residual + o   (residual 0 when absent).

    [dothoosh] "two-tower mechanism": the context tower is causal over the
    prompt and the committed tokens.

    Shapes: q_blk [B,S,Hq,d], k_blk/v_blk [B,S,Hkv,d], k_ctx/v_ctx
    [T_ctx,Hkv,d], ctx_start [B], ctx_len [B] (may be 0), residual
    [B,S,Hq,d] or None, active [B] or None.
    Returns (out [B,S,Hq,d], lse [B,S,Hq]) float64; rows of inactive
    sequences are NaN.
    """
    q = _f64(q_blk)
    kb, vb = _f64(k_blk), _f64(v_blk)
    kc, vc = _f64(k_ctx), _f64(v_ctx)
    B, S, Hq, d = q.shape
    Hkv = kb.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    out = np.full((B, S, Hq, d), np.nan)
    lse = np.full((B, S, Hq), np.nan)
    for b in range(B):
        if active is not None and not active[b]:
            continue
        st, n = int(ctx_start[b]), int(ctx_len[b])
        for h in range(Hq):
            g = h // group
            for s in range(S):
                keys = np.concatenate([kc[st:st + n, g, :], kb[b, :s + 1, g, :]], axis=0)
                vals = np.concatenate([vc[st:st + n, g, :], vb[b, :s + 1, g, :]], axis=0)
                sc = keys @ q[b, s, h, :] / np.sqrt(d)            # [n + s + 1]
                mx = sc.max()
                e = np.exp(sc - mx)
                z = e.sum()
                o = (e / z) @ vals
                lse[b, s, h] = mx + np.log(z)
                if residual is not None:
                    o = o + _f64(residual)[b, s, h, :]
                out[b, s, h, :] = o
    return out, lse


def kv_append(k_ctx, v_ctx, k_blk, v_blk, ctx_start, ctx_end, ctx_len, active=None):
    """Append a committed block's K/V to one layer's cache.

    For every active sequence b with ctx_len[b] + S <= ctx_end[b] - ctx_start[b]:
        k_ctx[ctx_start[b] + ctx_len[b] + s] = k_blk[b, s]   (s < S; V likewise)
    Every other cache row is left as it was.

    [dothoosh] "two-tower mechanism": the context tower keeps the per-layer KV
    cache of the prompt and the committed tokens.

    Returns (k_ctx', v_ctx', appended [B] bool) -- copies; the inputs are not
    modified.  The context lengths are advanced by ctx_advance.
    """
    kc = np.array(k_ctx, copy=True)
    vc = np.array(v_ctx, copy=True)
    kb, vb = np.asarray(k_blk), np.asarray(v_blk)
    B, S = kb.shape[0], kb.shape[1]
    appended = np.zeros(B, dtype=bool)
    for b in range(B):
        if active is not None and not active[b]:
            continue
        st, n = int(ctx_start[b]), int(ctx_len[b])
        if n + S > int(ctx_end[b]) - st:
            continue
        kc[st + n:st + n + S] = kb[b]
        vc[st + n:st + n + S] = vb[b]
        appended[b] = True
    return kc, vc, appended


def ctx_advance(block_size, ctx_start, ctx_end, ctx_len, active=None):
    """Grow every context that has room by one block: the length rule that
    goes with kv_append (same room test).  Returns (ctx_len' [B] int64,
    appended [B] bool)."""
    n = np.asarray(ctx_len, dtype=np.int64).copy()
    appended = np.zeros(n.shape[0], dtype=bool)
    for b in range(n.shape[0]):
        if active is not None and not active[b]:
            continue
        if n[b] + block_size <= int(ctx_end[b]) - int(ctx_start[b]):
            n[b] += block_size
            appended[b] = True
    return n, appended
