"""GPU parity of tt_confidence_unmask against the fp64 oracle: committed ids,
masks, predictions and counts bit-exact; confidences within the fp32 bound."""
import math

import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle
import synth

from .gpu_cases import DEV, np64, say

pytestmark = pytest.mark.gpu


def run_unmask(logits, tokens, masked, gamma, tau, step=0, mask_id=3, commit_step=None,
               row_stride=None, V=None):
    B, S = tokens.shape
    V = logits.shape[-1] if V is None else V
    stride = logits.shape[-1] if row_stride is None else row_stride
    ws = torch.empty(tt.unmask_workspace_size(B, S, V), dtype=torch.uint8, device=DEV)
    tok = tokens.clone().to(DEV, torch.int32)
    msk = masked.clone().to(DEV, torch.uint8)
    now = torch.full((B, S), 9, dtype=torch.uint8, device=DEV)
    conf = torch.zeros((B, S), dtype=torch.float32, device=DEV)
    pred = torch.zeros((B, S), dtype=torch.int32, device=DEV)
    cst = (torch.full((B, S), -1, dtype=torch.int8, device=DEV) if commit_step is None
           else commit_step.clone().to(DEV, torch.int8))
    nm = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    tt.confidence_unmask(B, S, V, logits, stride, gamma, tau, mask_id, step, tok, msk, ws,
                         committed_now=now, conf=conf, pred=pred, commit_step=cst, n_masked=nm)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), masked=msk.cpu().numpy(),
                committed_now=now.cpu().numpy(), conf=conf.cpu().numpy(),
                pred=pred.cpu().numpy(), commit_step=cst.cpu().numpy(),
                n_masked=nm.cpu().numpy())


def check(logits, tokens, masked, gamma, tau, step=0, what="", row_stride=None, V=None,
          seqs=None):
    say(what, tuple(logits.shape), logits.dtype, "gamma", gamma, "tau", tau)
    g = run_unmask(logits, tokens, masked, gamma, tau, step=step, row_stride=row_stride, V=V)
    B, S = tokens.shape
    V = logits.shape[-1] if V is None else V
    seqs = list(range(B)) if seqs is None else list(seqs)
    lg = np64(logits.reshape(B, S, -1)[seqs, :, :V])
    # the oracle gets gamma and tau as the library receives them (fp32)
    r = oracle.confidence_unmask(lg, tokens.numpy()[seqs], masked.numpy()[seqs],
                                 float(np.float32(gamma)), float(np.float32(tau)), 3,
                                 step, commit_step=np.full((len(seqs), S), -1))
    assert r["ambiguous"] == 0
    for key in ("tokens", "masked", "committed_now", "pred", "n_masked"):
        np.testing.assert_array_equal(g[key][seqs].astype(np.int64), r[key].astype(np.int64),
                                      err_msg=f"{what}: {key}")
    np.testing.assert_array_equal(g["commit_step"][seqs].astype(np.int64),
                                  r["commit_step"].astype(np.int64))
    m = masked.numpy()[seqs] > 0
    assert np.all(np.isnan(g["conf"][seqs][~m]))
    err = np.abs(g["conf"][seqs][m] - r["conf"][m])
    assert err.size == 0 or err.max() < 2e-5, f"{what}: conf err {err.max()}"
    return g, r


def _tokens(B, S, masked, V, seed=0):
    ids = synth.token_ids((B, S), V, seed)
    return torch.where(masked > 0, torch.full_like(ids, 3), ids)


# Tiny fp32 step: 16 slots with 10 masked, logits 16 x 1024 ~ N(0, 3), gamma 0.8.
def test_tiny_fp32_unmask():
    masked = synth.masked_subset(1, 16, 10, seed=1)
    logits = synth.normal((1, 16, 1024), 3.0, 11, torch.float32, DEV)
    check(logits, _tokens(1, 16, masked, 1024), masked, 0.8, 1.0, what="tiny fp32")


@pytest.mark.parametrize("gamma", [0.6, 0.8, 0.95])
@pytest.mark.parametrize("tau", [1.0, 0.1])
def test_vocab_131072_bf16(gamma, tau):
    B, S, V = 4, 16, 131072
    masked = torch.ones((B, S), dtype=torch.uint8)
    logits = synth.normal((B, S, V), 8.5 if tau == 1.0 else 0.85, 21, torch.bfloat16, DEV)
    g, r = check(logits, _tokens(B, S, masked, V), masked, gamma, tau, what="V=131072")
    assert g["committed_now"].sum() >= B


def test_headline_batch64_sampled():
    B, S, V = 64, 16, 131072
    masked = torch.ones((B, S), dtype=torch.uint8)
    logits = synth.normal((B, S, V), 8.5, 31, torch.bfloat16, DEV)
    check(logits, _tokens(B, S, masked, V), masked, 0.8, 1.0, what="64x16x131072",
          seqs=[0, 9, 33, 63])


def test_hand_built_rows():
    V = 2
    # U1: equal logits -> p = 1/2 exactly; inclusive threshold
    lg = torch.zeros((1, 3, V), dtype=torch.float32, device=DEV)
    masked = torch.ones((1, 3), dtype=torch.uint8)
    g, _ = check(lg, _tokens(1, 3, masked, V), masked, 0.5, 1.0, what="U1 gamma=.5")
    assert g["committed_now"].tolist() == [[1, 1, 1]] and np.all(g["conf"] == 0.5)
    g, _ = check(lg, _tokens(1, 3, masked, V), masked, 0.5 + 2 ** -20, 1.0, what="U1 above")
    assert g["committed_now"].tolist() == [[1, 0, 0]]
    # U4: ties -> lowest id; mask id may be predicted
    lg = torch.full((1, 4, 16), -2.0, dtype=torch.bfloat16, device=DEV)
    lg[0, 0, [9, 4, 12]] = 5.0
    lg[0, 1, 3] = 9.0
    lg[0, 2, [15, 14]] = 1.0
    masked = torch.tensor([[1, 1, 1, 0]], dtype=torch.uint8)
    g, _ = check(lg, _tokens(1, 4, masked, 16), masked, 0.8, 1.0, what="U4")
    assert g["pred"][0, :3].tolist() == [4, 3, 14] and g["pred"][0, 3] == -1


def test_identical_rows_below_gamma_commit_lowest_slot():
    B, S, V = 2, 16, 4096
    row = synth.normal((V,), 1.0, 41, torch.bfloat16, DEV)
    logits = row.expand(B, S, V).contiguous()
    masked = torch.ones((B, S), dtype=torch.uint8)
    masked[1, :5] = 0
    g, _ = check(logits, _tokens(B, S, masked, V), masked, 0.8, 1.0, what="identical rows")
    assert g["committed_now"][0].tolist() == [1] + [0] * 15
    assert g["committed_now"][1].tolist() == [0] * 5 + [1] + [0] * 10


# Rows whose p sits within 1e-7 of gamma: only the fp64 recheck decides them.
# V = 40003: rows not 16-byte aligned, and the recheck's full-row scan runs
# every loop of its strided read (head, four groups in flight, one group,
# scalar tail).
@pytest.mark.parametrize("side", [-1, 1])
@pytest.mark.parametrize("V", [1024, 40003])
def test_near_threshold_rows_decided_in_fp64(side, V):
    S = 8
    lg = torch.zeros((1, S, V), dtype=torch.float32)
    target = [0.8, 0.7, 0.9, 0.8, 0.5, 0.8, 0.3, 0.8]
    for s, p in enumerate(target):
        a = math.log(p * (V - 1) / (1 - p)) + side * 1e-7 * (s + 1)
        lg[0, s, (37 * s) % V] = a
    masked = torch.ones((1, S), dtype=torch.uint8)
    r0 = oracle.confidence_unmask(lg.double().numpy(), np.full((1, S), 3), masked.numpy(), 0.8,
                                  1.0, 3, 0)
    p = r0["conf"][0]
    gamma = float(np.float32(p[0]))         # gamma within one fp32 ulp of row 0's p
    g, r = check(lg.to(DEV), _tokens(1, S, masked, V), masked, gamma, 1.0, what="near gamma")
    assert np.any(np.abs(p - gamma) < 1e-6)


# No row reaches gamma, and the two most confident rows differ in fp64 p by
# about 1e-9: far below the error of an fp32 sum over the vocabulary, so only
# the decision kernel's fp64 recheck of the rows within its band of the best
# fp32 p can order them.  Every row has logit a at one token and 0 elsewhere
# (p = 1 / (1 + (V-1) e^-a) < gamma); the runner-up row also carries eps at
# one other token, which lowers its p by about p^2 e^-a eps.  The more
# confident row sits at the higher slot in sequence 0 and at the lower slot
# in sequence 1, so neither "lowest slot" nor a flipped fp32 order can pass
# by luck; the other rows have logit a - 0.5 (clearly lower p).
@pytest.mark.parametrize("V", [131072, 40003])
@pytest.mark.parametrize("eps_exp", [-11, -13])
def test_top_two_rows_ordered_in_fp64(V, eps_exp):
    B, S = 2, 16
    a, eps = 11.75, 2.0 ** eps_exp        # both exact in bf16
    lg = torch.zeros((B, S, V), dtype=torch.float32)
    for b in range(B):
        for s in range(S):
            lg[b, s, (101 * s + 7 + b) % V] = a - 0.5
    best, second = {0: (9, 3), 1: (2, 11)}, {}
    for b, (hi, lo) in best.items():
        lg[b, hi, (101 * hi + 7 + b) % V] = a
        lg[b, lo, (101 * lo + 7 + b) % V] = a
        lg[b, lo, (101 * lo + 500 + b) % V] = eps
        second[b] = lo
    logits = lg.to(torch.bfloat16)
    assert torch.equal(logits.float(), lg)
    masked = torch.ones((B, S), dtype=torch.uint8)
    r0 = oracle.confidence_unmask(lg.double().numpy(), np.full((B, S), 3), masked.numpy(), 0.8,
                                  1.0, 3, 0)
    for b, (hi, lo) in best.items():
        gap = r0["conf"][b, hi] - r0["conf"][b, lo]
        assert 1e-10 < gap < 1e-8 and r0["conf"][b].max() < 0.8, (b, gap)
    g, r = check(logits.to(DEV), _tokens(B, S, masked, V), masked, 0.8, 1.0,
                 what=f"top-2 rows 2^{eps_exp} apart, V={V}")
    for b, (hi, lo) in best.items():
        assert g["committed_now"][b].tolist() == [int(s == hi) for s in range(S)], b


def test_row_stride_and_scalar_path():
    B, S, V, stride = 2, 5, 1000, 1003        # stride not a multiple of 8 -> scalar loads
    logits = synth.normal((B * S * stride,), 3.0, 51, torch.bfloat16, DEV)
    masked = torch.ones((B, S), dtype=torch.uint8)
    masked[0, 2] = 0
    lg3 = logits.view(B, S, stride)
    check(lg3, _tokens(B, S, masked, V), masked, 0.3, 0.5, what="stride 1003", row_stride=stride,
          V=V)


def test_nothing_masked_and_deterministic():
    B, S, V = 3, 16, 2048
    masked = torch.zeros((B, S), dtype=torch.uint8)
    masked[2] = 1
    logits = synth.normal((B, S, V), 4.0, 61, torch.bfloat16, DEV)
    tok = _tokens(B, S, masked, V)
    a = run_unmask(logits, tok, masked, 0.8, 1.0)
    b = run_unmask(logits, tok, masked, 0.8, 1.0)
    for k in a:
        np.testing.assert_array_equal(np.nan_to_num(a[k], nan=-9), np.nan_to_num(b[k], nan=-9))
    assert a["n_masked"][:2].tolist() == [0, 0]
    np.testing.assert_array_equal(a["tokens"][:2], tok.numpy()[:2])
