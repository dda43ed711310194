"""GPU parity of tt_generate (multi-block generation: denoise, context-tower
append, EOS and room stops) against the fp64 oracle replaying the same
provider bytes: generated tokens, counts, stop reasons, context lengths and
the grown caches bit-exact."""
import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle
import synth

from .gpu_cases import DEV, assert_attn_close, np64, say

pytestmark = pytest.mark.gpu
MASK, EOS = 3, 7


class Provider:
    """Seeded synthetic stand-in for the rest of both towers.  Records what it
    gave (and the committed tokens it was shown) for the oracle's replay."""

    def __init__(self, B, S, Hq, Hkv, d, V, dtype, logit_std, eos_plan, seed):
        self.B, self.S, self.Hq, self.Hkv, self.d, self.V = B, S, Hq, Hkv, d, V
        self.dtype, self.std, self.eos_plan, self.seed = dtype, logit_std, eos_plan, seed
        self.qkv, self.lg, self.ctx, self.tokens = {}, {}, {}, {}
        self.last, self.ctx_prev = {}, {}

    def _fill(self, key, q, k, v):
        kind, blk, step, layer = key
        sd = self.seed + 100000 * kind + 1000 * blk + 50 * step + 5 * layer
        q.copy_(synth.normal(q.shape, 1.0, sd + 1, self.dtype, DEV))
        k.copy_(synth.normal(k.shape, 1.0, sd + 2, self.dtype, DEV))
        v.copy_(synth.normal(v.shape, 1.0, sd + 3, self.dtype, DEV))

    def layer_inputs(self, blk, step, layer, prev, q, k, v):
        self._fill((1, blk, step, layer), q, k, v)
        self.qkv[(blk, step, layer)] = tuple(np64(t) for t in (q, k, v))

    def logits(self, blk, step, last, lg):
        self.last[(blk, step)] = np64(last)
        x = synth.normal(lg.shape, self.std, self.seed + 7 * blk + 131 * step + 5, torch.float32, DEV)
        x[:, :, EOS] = -30.0                      # EOS only where planned
        for (b, bk, s) in self.eos_plan:          # a dominant EOS logit at (sequence, block, slot)
            if bk == blk:
                x[b, s, :] = 0.0
                x[b, s, EOS] = 60.0
        lg.copy_(x.to(lg.dtype))
        self.lg[(blk, step)] = np64(lg)

    def ctx_inputs(self, blk, layer, tokens, prev, q, k, v):
        self.tokens[(blk, layer)] = tokens.cpu().numpy().copy()
        if prev is not None:
            self.ctx_prev[(blk, layer)] = np64(prev)
        self._fill((2, blk, 0, layer), q, k, v)
        # the context tower's K/V depend on the committed tokens (an embedding)
        emb = (tokens.to(torch.float32) / 1024.0)[:, :, None, None]
        k.copy_((k.to(torch.float32) + emb).to(k.dtype))
        v.copy_((v.to(torch.float32) - emb).to(v.dtype))
        self.ctx[(blk, layer)] = tuple(np64(t) for t in (q, k, v))


def _run(B=3, S=16, Hq=8, Hkv=2, d=64, V=2048, NL=2, lens=(100, 0, 37), room=(3, 3, 3),
         n_blocks=3, steps=16, gamma=0.8, tau=1.0, seed=None, dtype=torch.bfloat16,
         logit_std=8.5, eos_plan=((0, 1, 5),), what="", stream=None):
    say("generate", what, dict(B=B, S=S, V=V, NL=NL, lens=lens, n_blocks=n_blocks, steps=steps,
                               tau=tau, seed=seed))
    lens = list(lens)
    cap = [l + r * S for l, r in zip(lens, room)]
    start = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    T = int(sum(cap))
    ctx_start = torch.tensor(start, dtype=torch.int64, device=DEV)
    ctx_end = torch.tensor(start + np.asarray(cap), dtype=torch.int64, device=DEV)
    ctx_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kc = [synth.normal((T, Hkv, d), 1.0, 900 + l, dtype, DEV) for l in range(NL)]
    vc = [synth.normal((T, Hkv, d), 1.0, 950 + l, dtype, DEV) for l in range(NL)]
    kc0 = [np64(x) for x in kc]
    vc0 = [np64(x) for x in vc]
    shape = tt.attn_shape(B, Hq, Hkv, d, S, dtype)
    ws = torch.empty(tt.generate_workspace_size(shape, NL, n_blocks, max(lens), V),
                     dtype=torch.uint8, device=DEV)
    out = torch.full((B, n_blocks * S), -5, dtype=torch.int32, device=DEV)
    n_gen = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    stop = torch.full((B,), -1, dtype=torch.int8, device=DEV)
    prov = Provider(B, S, Hq, Hkv, d, V, dtype, logit_std, eos_plan, 4242)
    if stream is not None:
        torch.cuda.synchronize()     # inputs were made on torch's current stream
    taken = tt.generate(shape, NL, n_blocks, steps, gamma, tau, MASK, EOS, V, kc, vc, ctx_start,
                        ctx_end, ctx_len, max(lens), prov, out, n_gen, ws, stop_reason=stop,
                        seed=seed, stream=stream)
    torch.cuda.synchronize()

    def ctx_inputs(blk, layer, tokens):
        np.testing.assert_array_equal(np.asarray(tokens), prov.tokens[(blk, layer)],
                                      err_msg=f"{what}: committed tokens of block {blk}")
        return prov.ctx[(blk, layer)]
    f32 = lambda x: float(np.float32(x))  # noqa: E731  (fp32, as the library receives them)
    r = oracle.generate(lambda blk, k, l: prov.qkv[(blk, k, l)], lambda blk, k: prov.lg[(blk, k)],
                        ctx_inputs, kc0, vc0, start, start + np.asarray(cap), np.asarray(lens), S,
                        n_blocks, f32(gamma), f32(tau), MASK, eos_token_id=EOS,
                        steps_per_block=steps, seed=seed)
    assert r["ambiguous"] == 0
    assert taken == r["blocks_taken"], what
    got = out.cpu().numpy().astype(np.int64)
    want = np.where(r["tokens"] < 0, -5, r["tokens"])
    np.testing.assert_array_equal(got, want, err_msg=f"{what}: tokens")
    assert n_gen.cpu().tolist() == r["n_generated"].tolist(), what
    assert stop.cpu().tolist() == r["stop"].tolist(), what
    assert ctx_len.cpu().tolist() == r["ctx_len"].tolist(), what
    for l in range(NL):
        np.testing.assert_array_equal(np64(kc[l]), r["k_ctx"][l], err_msg=f"{what}: k cache {l}")
        np.testing.assert_array_equal(np64(vc[l]), r["v_ctx"][l], err_msg=f"{what}: v cache {l}")
    # the attention inside the loop read the grown caches: the denoiser's last
    # layer at every step and the context tower's layers (seen by the next
    # layer's callback) match the oracle's, for the sequences that ran
    for blk, x in enumerate(r["denoise"]):
        for k, per_layer in enumerate(x["outputs"]):
            act = np.flatnonzero(x["n_masked_trace"][k] > 0)
            ro = per_layer[NL - 1][0][act]
            assert_attn_close(prov.last[(blk, k)][act], None, ro, None, dtype,
                              f"{what}: denoiser block {blk} step {k}")
        ran = np.flatnonzero(r["n_generated"] > blk * S)
        for l in range(1, NL):
            ro = r["ctx_outputs"][blk][l - 1][0][ran]
            assert_attn_close(prov.ctx_prev[(blk, l)][ran], None, ro, None, dtype,
                              f"{what}: context tower block {blk} layer {l - 1}")
    return r


# The pages' generation call: S = 16, steps_per_block = 16, gamma = 0.8, mask
# id 3, greedy and sampled at temperature 0.1 and 1; sequence 0 commits EOS in
# its second block.
@pytest.mark.parametrize("tau,seed", [(1.0, None), (0.1, 11), (1.0, 12)])
def test_generate_eos_and_blocks(tau, seed):
    r = _run(tau=tau, seed=seed, what=f"tau={tau} seed={seed}")
    assert r["stop"].tolist() == [1, 0, 0]
    assert r["n_generated"].tolist() == [32, 48, 48]


# Fewer steps than slots: the last allowed step commits the rest; flat
# logits make every step commit a single slot before it.
def test_generate_few_steps_final_commit():
    r = _run(steps=3, logit_std=0.5, eos_plan=(), what="steps=3")
    for x in r["denoise"]:
        assert x["steps_taken"] == 3 and x["masked"].sum() == 0


# A region with room for one block only: the sequence stops after its second
# block (its append found no room); the others go on.
def test_generate_room_stop():
    r = _run(room=(1, 3, 1), eos_plan=(), n_blocks=3, what="room")
    assert r["stop"].tolist() == [2, 0, 2]


# fp32 tower state, 4 query heads / 1 KV head, head dim 64 (the tiny workload's
# attention shape), S = 4, sampling.
def test_generate_fp32_small():
    _run(B=2, S=4, Hq=4, Hkv=1, d=64, V=1024, NL=1, lens=(128, 5), room=(4, 4), n_blocks=4,
         steps=4, tau=1.0, seed=3, dtype=torch.float32, logit_std=3.0, eos_plan=((1, 2, 0),),
         what="fp32 small")


# Every sequence stops at EOS in the first block: one block taken.
def test_generate_all_stop_early():
    r = _run(eos_plan=((0, 0, 1), (1, 0, 15), (2, 0, 0)), n_blocks=4, what="all EOS")
    assert r["blocks_taken"] == 1 and r["stop"].tolist() == [1, 1, 1]


# Generation on a stream other than torch's current one (sampled at the pages'
# temperature 0.1): every callback's copies run on the library's stream.
def test_generate_on_a_side_stream():
    r = _run(tau=0.1, seed=31, what="side stream", stream=torch.cuda.Stream())
    assert r["stop"].tolist() == [1, 0, 0]
