"""GPU parity of tt_sample_unmask (temperature sampling + commit rule) against
the fp64 oracle: drawn tokens, commits, masks and counts bit-exact; the
confidence within the fp32 bound."""
import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle
import synth
from oracle import sampling

from .gpu_cases import DEV, np64, say

pytestmark = pytest.mark.gpu


def f32(x):
    """A value as the library receives it (fp32: gamma, temperature), as the
    oracle's float."""
    return float(np.float32(x))


def run_sample(logits, tokens, masked, gamma, tau, seed, block, step=0, row_stride=None, V=None):
    B, S = tokens.shape
    V = logits.shape[-1] if V is None else V
    stride = logits.shape[-1] if row_stride is None else row_stride
    ws = torch.empty(tt.unmask_workspace_size(B, S, V), dtype=torch.uint8, device=DEV)
    tok = tokens.clone().to(DEV, torch.int32)
    msk = masked.clone().to(DEV, torch.uint8)
    now = torch.full((B, S), 9, dtype=torch.uint8, device=DEV)
    conf = torch.zeros((B, S), dtype=torch.float32, device=DEV)
    pred = torch.zeros((B, S), dtype=torch.int32, device=DEV)
    cst = torch.full((B, S), -1, dtype=torch.int8, device=DEV)
    nm = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    tt.sample_unmask(B, S, V, logits, stride, gamma, tau, seed, block, 3, step, tok, msk, ws,
                     committed_now=now, conf=conf, pred=pred, commit_step=cst, n_masked=nm)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), masked=msk.cpu().numpy(),
                committed_now=now.cpu().numpy(), conf=conf.cpu().numpy(),
                pred=pred.cpu().numpy(), commit_step=cst.cpu().numpy(),
                n_masked=nm.cpu().numpy())


def check(logits, tokens, masked, gamma, tau, seed, block, step=0, what="", row_stride=None,
          V=None, seqs=None):
    say(what, tuple(logits.shape), logits.dtype, "gamma", gamma, "tau", tau, "seed", seed,
        "block", block, "step", step)
    g = run_sample(logits, tokens, masked, gamma, tau, seed, block, step, row_stride, V)
    B, S = tokens.shape
    V = logits.shape[-1] if V is None else V
    seqs = list(range(B)) if seqs is None else list(seqs)
    lg = np64(logits.reshape(B, S, -1)[:, :, :V])
    # the oracle takes the whole batch (its row ids are b*S + s)
    r = oracle.confidence_unmask(lg, tokens.numpy(), masked.numpy(), f32(gamma), f32(tau), 3, step,
                                 commit_step=np.full((B, S), -1), sample=(seed, block))
    assert r["ambiguous"] == 0
    for key in ("tokens", "masked", "committed_now", "pred", "n_masked", "commit_step"):
        np.testing.assert_array_equal(g[key][seqs].astype(np.int64), r[key][seqs].astype(np.int64),
                                      err_msg=f"{what}: {key}")
    m = masked.numpy()[seqs] > 0
    assert np.all(np.isnan(g["conf"][seqs][~m]))
    err = np.abs(g["conf"][seqs][m] - r["conf"][seqs][m])
    assert err.size == 0 or err.max() < 2e-5, f"{what}: conf err {err.max()}"
    return g, r


def _tokens(B, S, masked, V, seed=0):
    ids = synth.token_ids((B, S), V, seed)
    return torch.where(masked > 0, torch.full_like(ids, 3), ids)


# Tiny fp32 step (16 slots, 10 masked, V = 1024, N(0, 3^2)) at tau = 1: with
# tau * 20 = 20 every token is a candidate, so the noise of all of them counts.
@pytest.mark.parametrize("tau", [1.0, 0.1])
def test_tiny_fp32(tau):
    masked = synth.masked_subset(1, 16, 10, seed=1)
    logits = synth.normal((1, 16, 1024), 3.0, 11, torch.float32, DEV)
    check(logits, _tokens(1, 16, masked, 1024), masked, 0.8, tau, 1234, 0, what="tiny fp32")


# The pages' generation settings (tau = 0.1, gamma = 0.8) and tau = 1 on the
# 131072-token vocabulary, bf16, several seeds / steps / blocks.
@pytest.mark.parametrize("tau,seed,block,step", [(0.1, 7, 0, 0), (0.1, 2**40 + 3, 5, 11),
                                                 (1.0, 99, 2, 3)])
def test_vocab_131072_bf16(tau, seed, block, step):
    B, S, V = 2, 16, 131072
    masked = torch.ones((B, S), dtype=torch.uint8)
    masked[1, ::3] = 0
    logits = synth.normal((B, S, V), 8.5, 40 + block, torch.bfloat16, DEV)
    check(logits, _tokens(B, S, masked, V), masked, 0.8, tau, seed, block, step,
          what="V=131072 bf16")


# Ragged vocabularies (slices with a partial tail; rows not 16-byte aligned)
# and a row stride larger than the vocabulary.
@pytest.mark.parametrize("V", [1, 2, 1000, 8191, 8193, 20001])
def test_ragged_vocab(V):
    B, S = 2, 4
    masked = torch.ones((B, S), dtype=torch.uint8)
    logits = synth.normal((B, S, V), 2.0, 50 + V, torch.bfloat16, DEV)
    check(logits, _tokens(B, S, masked, V), masked, 0.6, 0.5, 5, 1, what=f"V={V}")


def test_row_stride():
    B, S, V, W = 2, 8, 5000, 5120
    masked = torch.ones((B, S), dtype=torch.uint8)
    buf = synth.normal((B, S, W), 3.0, 60, torch.float32, DEV)
    check(buf, _tokens(B, S, masked, V), masked, 0.8, 0.7, 3, 0, what="row stride", row_stride=W,
          V=V)


# Planted near-ties of the perturbed scores: token 1's logit is set so that
# l_1 + tau G_1 lies within a few fp32 ulps of l_0 + tau G_0 (the noise taken
# from the oracle's generator for that slot), far below the fp32 decision
# band: the fp64 rescoring path must pick the oracle's token.  At V = 40003
# the pair sits mid-row and the rows are not 16-byte aligned, so the fp64 scan
# runs its head, its four-groups-in-flight loop, its one-group loop and its
# scalar tail.
@pytest.mark.parametrize("V", [64, 40003])
def test_planted_score_near_ties(V):
    B, S, tau, seed, block, step = 1, 8, 0.5, 77, 3, 2
    tau32 = f32(tau)
    lg = np.full((B, S, V), -30.0)
    pairs = []
    for s in range(S):
        i0 = 0 if V == 64 else 20000 + 37 * s
        g = sampling.gumbel_noise(seed, s, step, block, V)
        lg[0, s, i0] = 1.0
        target = 1.0 + tau32 * (g[i0] - g[i0 + 1])
        l1 = np.float32(target)
        # step to the float32 neighbour on the side the slot asks for
        for _ in range(s % 3):
            l1 = np.nextafter(l1, np.float32(np.inf) if s % 2 else np.float32(-np.inf))
        lg[0, s, i0 + 1] = float(l1)
        pairs.append({i0, i0 + 1})
    logits = torch.tensor(lg, dtype=torch.float32, device=DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    g, r = check(logits, _tokens(B, S, masked, V), masked, 0.8, tau, seed, block, step,
                 what=f"planted near-ties V={V}")
    assert all(int(t) in pairs[s] for s, t in enumerate(r["pred"][0].tolist()))


# Planted confidences next to gamma (V = 2, logits (a, 0), p = sigmoid(a/tau)
# for the drawn token 0): the fp64 recheck of p decides.
def test_planted_confidence_near_gamma():
    B, S, V, tau = 1, 16, 2, 1.0
    gamma = 0.8
    a = np.log(gamma / (1 - gamma))
    lg = np.zeros((B, S, V), dtype=np.float32)
    for s in range(S):
        x = np.float32(a)
        for _ in range(s % 4):
            x = np.nextafter(x, np.float32(np.inf) if s % 2 else np.float32(-np.inf))
        lg[0, s, 0] = x
    logits = torch.tensor(lg, device=DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    check(logits, _tokens(B, S, masked, V), masked, gamma, tau, 5, 0, what="near gamma")


# Flat rows: every token of the vocabulary is a candidate at every slice.
def test_flat_rows():
    B, S, V = 1, 4, 40000
    logits = torch.zeros((B, S, V), dtype=torch.bfloat16, device=DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    check(logits, _tokens(B, S, masked, V), masked, 0.8, 0.1, 11, 0, what="flat rows")


# gamma <= 0 commits every masked slot (the generation loop's last step).
def test_gamma_nonpositive_commits_all():
    B, S, V = 2, 16, 4096
    logits = synth.normal((B, S, V), 1.0, 70, torch.bfloat16, DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    masked[0, :5] = 0
    g, _ = check(logits, _tokens(B, S, masked, V), masked, float("-inf"), 0.1, 1, 0,
                 what="gamma -inf")
    assert g["masked"].sum() == 0


# Full size, the launch the benchmark times: 64 x 16 slots, V = 131072,
# N(0, 8.5^2) logits, tau = 0.1 -- checked on a sample of sequences (the
# oracle computes the whole batch's row ids but only those sequences' rows).
def test_headline_sampled():
    B, S, V = 64, 16, 131072
    logits = synth.normal((B, S, V), 8.5, 1234 + 70, torch.bfloat16, DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    toks = _tokens(B, S, masked, V)
    say("headline sampling 64x16x131072")
    g = run_sample(logits, toks, masked, 0.8, 0.1, 2024, 0)
    seqs = [0, 21, 63]
    for b in seqs:
        lg = np64(logits[b:b + 1])
        # row ids of sequence b: b*S + s -> replay with the oracle's row ids
        preds, confs = [], []
        for s in range(S):
            p, c, margin = sampling.row_sample(lg[0, s], f32(0.1), 2024, b * S + s, 0, 0)
            assert margin > 1e-12
            preds.append(p)
            confs.append(c)
        assert g["pred"][b].tolist() == preds
        assert np.abs(g["conf"][b] - np.array(confs)).max() < 2e-5
        ok = [c >= f32(0.8) for c in confs]
        want = [s for s in range(S) if ok[s]] or [int(np.argmax(confs))]
        assert sorted(np.flatnonzero(g["committed_now"][b]).tolist()) == want


def test_sample_deterministic_and_seed_dependent():
    B, S, V = 4, 16, 32768
    logits = synth.normal((B, S, V), 1.0, 80, torch.bfloat16, DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    toks = _tokens(B, S, masked, V)
    a = run_sample(logits, toks, masked, 0.8, 1.0, 5, 0)
    b = run_sample(logits, toks, masked, 0.8, 1.0, 5, 0)
    c = run_sample(logits, toks, masked, 0.8, 1.0, 6, 0)
    assert all(np.array_equal(a[k], b[k]) for k in a if k != "conf")
    assert np.array_equal(a["conf"], b["conf"])
    assert (a["pred"] != c["pred"]).mean() > 0.5
