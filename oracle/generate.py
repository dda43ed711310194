"""fp64 definition of multi-block generation: denoise a block, let the context
tower consume it, move to the next block, stop at EOS (test infrastructure;
see the package header).

Pages followed (tags defined in oracle/__init__.py):
  * [news] "training and inference" code example: the generation call takes
    max_new_tokens=128, block_size=16, steps_per_block=16, mask_token_id=3,
    temperature=0.1, confidence_threshold=0.8 and eos_token_id.
  * [dothoosh] "two-tower mechanism": generation goes block by block; each
    block starts as [MASK] tokens and is refined over T steps until final;
    the context tower runs causally over the prompt and the committed tokens
    and keeps every layer's KV cache.

Readings where the pages are silent:
  * whole blocks are generated (n_blocks = ceil(max_new_tokens / S)); a
    sequence stops after the block in which it commits eos_token_id (the
    tokens after it in that block are kept; the caller cuts at EOS), or when
    its cache region has no room for the next block;
  * a block is final when the context tower takes it: the last allowed step
    (steps_per_block, default S) commits every slot still masked;
  * the context tower takes a block through every attention layer in order
    (in-block causal attention over the grown context, block K/V appended),
    then every such context grows by S;
  * with sampling, the noise of block k uses block index k in its counter.
"""

import numpy as np

from .context import ctx_advance, ctx_block_attn, kv_append
from .unmask import denoise_block


def generate(denoise_inputs, denoise_logits, ctx_inputs, k_ctx_layers, v_ctx_layers,
             ctx_start, ctx_end, ctx_len, block_size, n_blocks, gamma, temperature,
             mask_token_id, eos_token_id=None, steps_per_block=None, seed=None,
             ada_w=None, ada_bias=None, ada_table=None):
    """The generation loop over n_blocks blocks of block_size slots.

    denoise_inputs(blk, step, layer) -> (q, k_blk, v_blk) of the denoiser,
    denoise_logits(blk, step) -> logits [B,S,V],
    ctx_inputs(blk, layer, tokens) -> (q, k_blk, v_blk) of the context tower
    for the committed block `tokens` [B,S]
    (the rest of both towers; the tests replay the bytes a GPU provider gave).
    k_ctx_layers/v_ctx_layers: per-layer caches [T, Hkv, d]; ctx_start,
    ctx_end (reserved regions), ctx_len: [B].  seed: None for the argmax
    prediction, else temperature sampling with that seed.

    For block k while some sequence is unfinished:
      1. the unfinished sequences' blocks start fully masked; denoise_block
         (up to steps_per_block steps, the last one committing every masked
         slot, sampling with block index k when seeded);
      2. their tokens are written to out[b, k*S:(k+1)*S], n_generated += S;
      3. for each layer: (q, k, v) = ctx_inputs(k, layer, tokens);
         ctx_block_attn over the current cache, kv_append of (k, v); then
         ctx_advance for every unfinished sequence;
      4. a sequence whose block holds eos_token_id stops (stop = 1), one
         whose cache had no room stops (stop = 2).
    Returns dict(tokens [B, n_blocks*S] (-1 where not generated),
    n_generated [B], stop [B] (0: all blocks generated), blocks_taken,
    ctx_len [B], k_ctx / v_ctx (lists of caches), denoise (per block: the
    denoise_block result), ctx_outputs (per block, per layer: (out, lse)),
    ambiguous).
    """
    kc = [np.array(x, copy=True) for x in k_ctx_layers]
    vc = [np.array(x, copy=True) for x in v_ctx_layers]
    lens = np.asarray(ctx_len, dtype=np.int64).copy()
    B, S = len(lens), int(block_size)
    finished = np.zeros(B, dtype=bool)
    stop = np.zeros(B, dtype=np.int64)
    out = np.full((B, n_blocks * S), -1, dtype=np.int64)
    n_gen = np.zeros(B, dtype=np.int64)
    steps = S if steps_per_block is None else int(steps_per_block)
    per_block, ctx_outs = [], []
    ambiguous = 0
    taken = 0
    for blk in range(n_blocks):
        active = ~finished
        if not active.any():
            break
        tok = np.full((B, S), mask_token_id, dtype=np.int64)
        msk = np.repeat(active[:, None], S, axis=1).astype(np.uint8)
        r = denoise_block(lambda k, l: denoise_inputs(blk, k, l),
                          lambda k: denoise_logits(blk, k), kc, vc, ctx_start, lens,
                          tok, msk, gamma, temperature, mask_token_id, max_steps=steps,
                          ada_w=ada_w, ada_bias=ada_bias, ada_table=ada_table,
                          sample=None if seed is None else (seed, blk), finish_block=True)
        per_block.append(r)
        ambiguous += r["ambiguous"]
        tok = r["tokens"]
        for b in np.flatnonzero(active):
            out[b, blk * S:(blk + 1) * S] = tok[b]
            n_gen[b] += S
        layer_outs = []
        act_u8 = active.astype(np.uint8)
        for layer in range(len(kc)):
            q, kb, vb = ctx_inputs(blk, layer, tok)
            layer_outs.append(ctx_block_attn(q, kb, vb, kc[layer], vc[layer], ctx_start, lens,
                                             active=act_u8))
            kc[layer], vc[layer], _ = kv_append(kc[layer], vc[layer], kb, vb, ctx_start,
                                                ctx_end, lens, act_u8)
        ctx_outs.append(layer_outs)
        lens, appended = ctx_advance(S, ctx_start, ctx_end, lens, act_u8)
        for b in np.flatnonzero(active):
            if eos_token_id is not None and np.any(tok[b] == eos_token_id):
                finished[b] = True
                stop[b] = 1
            elif not appended[b]:
                finished[b] = True
                stop[b] = 2
        taken = blk + 1
    return dict(tokens=out, n_generated=n_gen, stop=stop, blocks_taken=taken, ctx_len=lens,
                k_ctx=kc, v_ctx=vc, denoise=per_block, ctx_outputs=ctx_outs,
                ambiguous=ambiguous)
