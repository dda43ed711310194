"""fp64 definition of confidence unmasking and of the block denoising loop
(test infrastructure; see the package header).

Pages followed (tags defined in oracle/__init__.py):
  * [keyframe] "key points" item 3 and "full analysis": the denoiser predicts
    all masked slots of a 16-token block at once, commits the tokens it is
    confident about step by step, and re-masks the undetermined rest.
  * [dothoosh] "two-tower mechanism": each block starts as [MASK] tokens and is
    refined over T steps until its tokens are final; benchmark paragraph:
    lowering the confidence threshold gamma commits more tokens per step.
  * [news] "training and inference" code example: block_size=16,
    steps_per_block=16, mask_token_id=3, temperature=0.1,
    confidence_threshold=0.8.
  * [modelcard] "good to know" and "differentiators": confidence unmasking at
    gamma=0.8 commits several tokens per iteration.

Readings where the pages are silent:
  * confidence = the largest softmax probability of the row, computed as
    softmax(l / tau); the prediction is the argmax, lowest token id on ties;
  * commit every masked slot with p >= gamma (inclusive); if none qualifies,
    commit exactly the single most confident slot (lowest position on ties),
    so that S steps always finish an S-slot block;
  * committed slots are final; the uncommitted masked slots are written back
    as mask_token_id; the mask id itself may be predicted (masked state lives
    in the bitmap, not in the token value);
  * timestep of a step = (masked slots at the step's start) / S.
"""

import math

import numpy as np

from .attention import adaln_single, block_attn, timestep_embedding
from .sampling import row_sample

# Decisions whose fp64 margin is nonzero but below this are reported as
# ambiguous: two correct fp64 evaluations could take them either way.  Exact
# equalities (identical rows, p exactly equal to gamma) are not ambiguous:
# every deterministic evaluation reproduces them, and the stated rules
# (inclusive threshold, lowest slot) settle them.
AMBIGUOUS_MARGIN = 1e-12


def row_confidence(row, temperature):
    """(pred, p) for one logit row: pred = lowest index of the maximum,
    p = 1 / sum_v exp((l_v - max) / tau)  (the probability of pred under
    softmax(l / tau)); the sum is exactly rounded (math.fsum)."""
    x = np.asarray(row, dtype=np.float64)
    m = x.max()
    pred = int(np.flatnonzero(x == m)[0])
    z = math.fsum(np.exp((x - m) / float(temperature)).tolist())
    return pred, 1.0 / z


def confidence_unmask(logits, tokens, masked, gamma, temperature,
                      mask_token_id, step, commit_step=None, sample=None,
                      commit_all=False):
    """One unmasking pass over a batch of blocks.

    logits [B,S,V], tokens [B,S] int, masked [B,S] bool/uint8 (slots still
    masked on entry), commit_step [B,S] int or None.

    For every sequence b, over its masked slots s: (pred_s, p_s) from
    row_confidence; C = {s : p_s >= gamma}; if C is empty and some slot is
    masked, C = {the slot of largest p, lowest s on ties}.  Slots in C take
    token pred_s, leave the mask and record commit_step = step; the other
    masked slots get mask_token_id.

    sample = (seed, block): temperature sampling instead of the argmax --
    (pred_s, p_s) from sampling.row_sample with row id b*S + s (the
    perturbed-score margins below AMBIGUOUS_MARGIN * (1 + |max|) are counted
    as ambiguous too).  commit_all: every masked slot is committed (the last
    step a block is allowed).

    Returns a dict of new arrays: tokens, masked (uint8), committed_now
    (uint8), conf (float64, NaN where not masked on entry), pred (int64, -1
    where not masked on entry), commit_step (or None), n_masked [B], and
    ambiguous (number of decisions whose nonzero fp64 margin is below
    AMBIGUOUS_MARGIN).
    """
    lg = np.asarray(logits)
    B, S, _ = lg.shape
    tok = np.array(tokens, dtype=np.int64, copy=True)
    msk = np.array(masked, dtype=np.uint8, copy=True)
    cstep = None if commit_step is None else np.array(commit_step, dtype=np.int64, copy=True)
    now = np.zeros((B, S), dtype=np.uint8)
    conf = np.full((B, S), np.nan)
    pred = np.full((B, S), -1, dtype=np.int64)
    ambiguous = 0
    g = float(gamma)
    for b in range(B):
        slots = [s for s in range(S) if msk[b, s]]
        for s in slots:
            if sample is None:
                pred[b, s], conf[b, s] = row_confidence(lg[b, s], temperature)
            else:
                pred[b, s], conf[b, s], margin = row_sample(lg[b, s], temperature, sample[0],
                                                            b * S + s, step, sample[1])
                scale = 1.0 + abs(float(np.max(lg[b, s])))
                ambiguous += int(0.0 < margin < AMBIGUOUS_MARGIN * scale)
        chosen = [s for s in slots if conf[b, s] >= g or commit_all]
        ambiguous += sum(1 for s in slots if 0.0 < abs(conf[b, s] - g) < AMBIGUOUS_MARGIN)
        if not chosen and slots:
            best = max(conf[b, s] for s in slots)
            top = min(s for s in slots if conf[b, s] == best)
            chosen = [top]
            ambiguous += sum(1 for s in slots
                             if 0.0 < best - conf[b, s] < AMBIGUOUS_MARGIN)
        for s in slots:
            if s in chosen:
                tok[b, s] = pred[b, s]
                msk[b, s] = 0
                now[b, s] = 1
                if cstep is not None:
                    cstep[b, s] = step
            else:
                tok[b, s] = mask_token_id
    return dict(tokens=tok, masked=msk, committed_now=now, conf=conf, pred=pred,
                commit_step=cstep, n_masked=msk.sum(axis=1).astype(np.int64),
                ambiguous=ambiguous)


def denoise_block(layer_inputs, step_logits, k_ctx_layers, v_ctx_layers,
                  ctx_start, ctx_len, tokens, masked, gamma, temperature,
                  mask_token_id, max_steps=None, ada_w=None, ada_bias=None,
                  ada_table=None, commit_step=None, sample=None,
                  finish_block=False):
    """The block denoising loop, replaying the bytes a step provider gave.

    [dothoosh] "two-tower mechanism": a block of [MASK] tokens is refined over
    up to T steps until final; [news] code example: steps_per_block = block
    size = 16.  For step k < max_steps (default S), while any slot is masked:
      1. t_b = n_masked_b / S; ada = adaln_single(timestep_embedding(t), ...)
         when adaLN weights are given (else identity modulation);
      2. for each layer l: (q, k_blk, v_blk) = layer_inputs(k, l);
         out_l = block_attn(... layer l's context KV ..., shift/scale/gate of
         layer l, residual None, active = n_masked > 0);
      3. logits = step_logits(k); confidence_unmask(...).
    Sequences with nothing masked are inactive (no attention rows, no
    unmasking).  Slots still masked after max_steps stay masked -- unless
    finish_block, when the last allowed step commits every masked slot.
    sample = (seed, block) selects temperature sampling (confidence_unmask).

    Returns dict(tokens, masked, commit_step, steps_taken, n_masked_trace
    [steps+1, B], outputs [step][layer] (out, lse), ambiguous).
    """
    tok = np.array(tokens, dtype=np.int64, copy=True)
    msk = np.array(masked, dtype=np.uint8, copy=True)
    B, S = tok.shape
    cstep = (np.full((B, S), -1, dtype=np.int64) if commit_step is None
             else np.array(commit_step, dtype=np.int64, copy=True))
    n_layers = len(k_ctx_layers)
    steps = S if max_steps is None else int(max_steps)
    n_trace = [msk.sum(axis=1).astype(np.int64)]
    outputs = []
    ambiguous = 0
    taken = 0
    for k in range(steps):
        n_m = msk.sum(axis=1)
        if n_m.sum() == 0:
            break
        active = n_m > 0
        shift = scale = gate = None
        ada = None
        if ada_w is not None:
            emb = timestep_embedding(n_m.astype(np.float64) / S)
            ada = adaln_single(emb, ada_w, ada_bias, ada_table)
        per_layer = []
        for layer in range(n_layers):
            q, kb, vb = layer_inputs(k, layer)
            if ada is not None:
                shift, scale, gate = ada[layer, 0], ada[layer, 1], ada[layer, 2]
            per_layer.append(block_attn(q, kb, vb, k_ctx_layers[layer],
                                        v_ctx_layers[layer], ctx_start, ctx_len,
                                        shift=shift, scale=scale, gate=gate,
                                        active=active))
        outputs.append(per_layer)
        r = confidence_unmask(step_logits(k), tok, msk, gamma, temperature,
                              mask_token_id, k, cstep, sample=sample,
                              commit_all=finish_block and k == steps - 1)
        tok, msk, cstep = r["tokens"], r["masked"], r["commit_step"]
        ambiguous += r["ambiguous"]
        n_trace.append(r["n_masked"])
        taken = k + 1
    return dict(tokens=tok, masked=msk, commit_step=cstep, steps_taken=taken,
                n_masked_trace=np.stack(n_trace), outputs=outputs,
                ambiguous=ambiguous)
