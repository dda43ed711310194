"""GPU parity of the whole denoising loop (tt_denoise_block) against the
oracle's replay of the same step-provider bytes."""
import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle
import synth

from .gpu_cases import DEV, TOL, np64, say

pytestmark = pytest.mark.gpu


class RecordedProvider:
    """Synthetic rest-of-the-denoiser: seeded q/k/v per (step, layer) and
    logits per step, copied into the library's buffers; keeps every layer's
    output of every step (layer l's arrives as prev_out of layer l + 1, the
    last layer's as last_out of the logits call)."""

    def __init__(self, B, S, Hq, Hkv, d, V, n_layers, steps, dtype, logit_std, seed):
        self.qkv = {}
        self.lg = {}
        for k in range(steps):
            for l in range(n_layers):
                s0 = seed + 1000 * k + 10 * l
                self.qkv[(k, l)] = (synth.normal((B, S, Hq, d), 1.0, s0 + 1, dtype, DEV),
                                    synth.normal((B, S, Hkv, d), 1.0, s0 + 2, dtype, DEV),
                                    synth.normal((B, S, Hkv, d), 1.0, s0 + 3, dtype, DEV))
            self.lg[k] = synth.normal((B, S, V), logit_std, seed + 1000 * k + 7, dtype, DEV)
        self.outs = {}
        self.n_layers = n_layers

    def layer_inputs(self, step, layer, prev_out, q, kb, vb):
        if layer > 0:
            self.outs[(step, layer - 1)] = prev_out.clone()
        a, b, c = self.qkv[(step, layer)]
        q.copy_(a)
        kb.copy_(b)
        vb.copy_(c)

    def logits(self, step, last_out, lg):
        self.outs[(step, self.n_layers - 1)] = last_out.clone()
        lg.copy_(self.lg[step])


def _run(B, S, Hq, Hkv, d, V, n_layers, lens, n_masked, dtype, logit_std, gamma, tau, ada,
         seed, max_steps=None, stream=None):
    say("denoise", dict(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, V=V, layers=n_layers, dtype=dtype))
    max_steps = S if max_steps is None else max_steps
    total = sum(lens)
    start = torch.tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]), dtype=torch.int64, device=DEV)
    clen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kc = [synth.normal((max(total, 1), Hkv, d), 1.0, seed + 50 + l, dtype, DEV) for l in range(n_layers)]
    vc = [synth.normal((max(total, 1), Hkv, d), 1.0, seed + 60 + l, dtype, DEV) for l in range(n_layers)]
    masked = synth.masked_subset(B, S, n_masked, seed=seed)
    tokens = torch.where(masked > 0, torch.full((B, S), 3, dtype=torch.int32),
                         synth.token_ids((B, S), V, seed))
    W = Hq * d
    ada_w = ada_b = ada_t = None
    if ada:
        ada_w = synth.normal((256, 3 * W), 0.05, seed + 70, torch.bfloat16, DEV)
        ada_b = synth.normal((3 * W,), 0.1, seed + 71, torch.float32, DEV)
        ada_t = synth.normal((n_layers, 3, W), 0.1, seed + 72, torch.float32, DEV)
    prov = RecordedProvider(B, S, Hq, Hkv, d, V, n_layers, max_steps, dtype, logit_std, seed)
    shape = tt.attn_shape(B, Hq, Hkv, d, S, dtype)
    ws = torch.empty(tt.denoise_workspace_size(shape, n_layers, max(lens), V), dtype=torch.uint8,
                     device=DEV)
    tok = tokens.to(DEV)
    msk = masked.to(DEV)
    cst = torch.full((B, S), -1, dtype=torch.int8, device=DEV)
    if stream is not None:
        torch.cuda.synchronize()     # inputs were made on torch's current stream
    taken = tt.denoise_block(shape, n_layers, max_steps, gamma, tau, 3, V, kc, vc, start, clen,
                             max(lens), prov, tok, msk, ws, commit_step=cst, ada_w=ada_w,
                             ada_bias=ada_b, ada_table=ada_t, stream=stream)
    torch.cuda.synchronize()
    r = oracle.denoise_block(
        lambda k, l: tuple(np64(t) for t in prov.qkv[(k, l)]), lambda k: np64(prov.lg[k]),
        [np64(t) for t in kc], [np64(t) for t in vc], start.cpu().numpy(), clen.cpu().numpy(),
        tokens.numpy(), masked.numpy(), float(np.float32(gamma)), float(np.float32(tau)), 3,
        max_steps=max_steps,
        ada_w=None if ada_w is None else np64(ada_w),
        ada_bias=None if ada_b is None else np64(ada_b),
        ada_table=None if ada_t is None else np64(ada_t))
    assert r["ambiguous"] == 0
    assert taken == r["steps_taken"]
    np.testing.assert_array_equal(tok.cpu().numpy(), r["tokens"])
    np.testing.assert_array_equal(msk.cpu().numpy(), r["masked"])
    np.testing.assert_array_equal(cst.cpu().numpy().astype(np.int64), r["commit_step"])
    tol = TOL[dtype]
    for k in range(taken):
        for l in range(n_layers):
            ref_out = r["outputs"][k][l][0]
            act = ~np.isnan(ref_out[:, 0, 0, 0])
            got = np64(prov.outs[(k, l)])[act]
            err = np.abs(got - ref_out[act]).max()
            assert err <= tol["max_abs"], f"step {k} layer {l}: attention max abs {err}"
    return taken, r


# The tiny fp32 step run to completion: batch 1, 1 layer, 4/1 heads, d 64,
# context 128, S 16 with 10 masked, logits 16 x 1024 ~ N(0, 3), gamma 0.8.
def test_tiny_fp32_loop():
    taken, r = _run(1, 16, 4, 1, 64, 1024, 1, [128], 10, torch.float32, 3.0, 0.8, 1.0,
                    ada=False, seed=1)
    assert r["masked"].sum() == 0 and taken <= 10


def test_bf16_loop_with_adaln():
    taken, r = _run(3, 16, 32, 2, 128, 4096, 2, [700, 0, 1500], 16, torch.bfloat16, 6.0, 0.8,
                    1.0, ada=True, seed=2)
    assert r["masked"].sum() == 0


def test_bf16_loop_stops_at_max_steps():
    taken, r = _run(2, 16, 8, 2, 64, 512, 1, [64, 33], 16, torch.bfloat16, 0.5, 0.99, 1.0,
                    ada=True, seed=3, max_steps=5)
    assert taken == 5 and r["masked"].sum() == 2 * (16 - 5)


def test_callback_error_reports_status():
    class Bad(RecordedProvider):
        def logits(self, step, last_out, lg):
            raise ValueError("boom")
    B, S, Hq, Hkv, d, V = 1, 4, 4, 1, 64, 64
    prov = Bad(B, S, Hq, Hkv, d, V, 1, 4, torch.float32, 1.0, 5)
    shape = tt.attn_shape(B, Hq, Hkv, d, S, torch.float32)
    kc = synth.normal((8, Hkv, d), 1.0, 1, torch.float32, DEV)
    ws = torch.empty(tt.denoise_workspace_size(shape, 1, 8, V), dtype=torch.uint8, device=DEV)
    tok = torch.full((B, S), 3, dtype=torch.int32, device=DEV)
    msk = torch.ones((B, S), dtype=torch.uint8, device=DEV)
    with pytest.raises(tt.TTError) as ei:
        tt.denoise_block(shape, 1, 4, 0.8, 1.0, 3, V, [kc], [kc],
                         torch.zeros(1, dtype=torch.int64, device=DEV),
                         torch.full((1,), 8, dtype=torch.int32, device=DEV), 8, prov, tok, msk, ws)
    assert ei.value.status == tt.TT_ERR_CALLBACK and "boom" in str(ei.value)
    assert int(msk.sum()) == S       # state of the last completed step (none)


# Block-size sweep of the full loop (the ctx-32768 sweep's S and gamma grid at
# a size the oracle replays in seconds): every step's commits, the final ids
# and masks, commit steps and step count must equal the oracle's.
@pytest.mark.parametrize("S", [4, 16, 64])
@pytest.mark.parametrize("gamma", [0.6, 0.8, 0.95])
def test_block_size_gamma_sweep(S, gamma):
    lens = [1500, 263] if S < 64 else [700, 129]
    taken, r = _run(2, S, 32, 2, 128, 2048, 1, lens, S, torch.bfloat16, 7.0, gamma, 1.0,
                    ada=True, seed=100 + S + int(100 * gamma))
    assert r["masked"].sum() == 0 and taken <= S


# The loop on a stream other than torch's current one: the provider's copies
# (and the outputs it keeps) must be ordered with the library's launches on
# that stream, so the results still equal the oracle's replay.
def test_loop_on_a_side_stream():
    side = torch.cuda.Stream()
    taken, r = _run(3, 16, 32, 2, 128, 4096, 3, [900, 64, 2100], 16, torch.bfloat16, 6.0, 0.8,
                    1.0, ada=True, seed=21, stream=side)
    assert r["masked"].sum() == 0


# Stop and resume: the loop stopped after j steps and continued with
# tt_denoise_block_resume from step j reaches the uninterrupted run's state
# bit for bit (ids, masks, commit steps, steps in total), with the argmax
# prediction and with temperature sampling (whose noise counters and
# commit_step use the absolute step).  The uninterrupted run itself equals
# the oracle's replay.
@pytest.mark.parametrize("seed,tau", [(None, 1.0), (77, 0.1)])
@pytest.mark.parametrize("j", [1, 5, 9])
def test_stop_and_resume(seed, tau, j):
    B, S, Hq, Hkv, d, V, NL = 3, 16, 32, 2, 128, 4096, 2
    lens = [700, 0, 1500]
    say("stop/resume", dict(j=j, seed=seed, tau=tau))
    start = torch.tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]), dtype=torch.int64, device=DEV)
    clen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kc = [synth.normal((sum(lens), Hkv, d), 1.0, 500 + l, torch.bfloat16, DEV) for l in range(NL)]
    vc = [synth.normal((sum(lens), Hkv, d), 1.0, 510 + l, torch.bfloat16, DEV) for l in range(NL)]
    W = Hq * d
    ada = dict(ada_w=synth.normal((256, 3 * W), 0.05, 520, torch.bfloat16, DEV),
               ada_bias=synth.normal((3 * W,), 0.1, 521, torch.float32, DEV),
               ada_table=synth.normal((NL, 3, W), 0.1, 522, torch.float32, DEV))
    masked0 = synth.masked_subset(B, S, 13, seed=523)
    tokens0 = torch.where(masked0 > 0, torch.full((B, S), 3, dtype=torch.int32),
                          synth.token_ids((B, S), V, 524))
    prov = RecordedProvider(B, S, Hq, Hkv, d, V, NL, S, torch.bfloat16, 6.0, 530)
    shape = tt.attn_shape(B, Hq, Hkv, d, S, torch.bfloat16)
    ws = torch.empty(tt.denoise_workspace_size(shape, NL, max(lens), V), dtype=torch.uint8,
                     device=DEV)

    def run(first, n, tok, msk, cst):
        return tt.denoise_block_resume(shape, NL, first, n, 0.8, tau, 3, V, kc, vc, start, clen,
                                       max(lens), prov, tok, msk, ws, commit_step=cst, seed=seed,
                                       block_index=2, **ada)

    def state():
        return (tokens0.to(DEV), masked0.to(DEV),
                torch.full((B, S), -1, dtype=torch.int8, device=DEV))
    a = state()
    taken_a = run(0, S, *a)
    b = state()
    taken_b = run(0, j, *b)
    taken_b += run(j, S - j, *b)
    torch.cuda.synchronize()
    for x, y, name in zip(a, b, ("tokens", "masked", "commit_step")):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy(), err_msg=name)
    assert taken_a == taken_b and int(a[1].sum()) == 0
    r = oracle.denoise_block(
        lambda k, l: tuple(np64(t) for t in prov.qkv[(k, l)]), lambda k: np64(prov.lg[k]),
        [np64(t) for t in kc], [np64(t) for t in vc], start.cpu().numpy(), clen.cpu().numpy(),
        tokens0.numpy(), masked0.numpy(), float(np.float32(0.8)), float(np.float32(tau)), 3,
        sample=None if seed is None else (seed, 2),
        **{k: np64(v) for k, v in ada.items()})
    assert r["ambiguous"] == 0 and r["steps_taken"] == taken_a
    np.testing.assert_array_equal(a[0].cpu().numpy(), r["tokens"])
    np.testing.assert_array_equal(a[2].cpu().numpy().astype(np.int64), r["commit_step"])
