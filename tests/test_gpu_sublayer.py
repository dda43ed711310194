"""GPU parity of the weighted adaLN-single attention sublayer through the C
ABI: tt_ln_modulate, tt_qkv_proj and tt_out_proj each against the fp64
oracle fed exactly the bytes the GPU consumed, and the composite
tt_adaln_attn_sublayer equal, bit for bit, to the chain of those calls and
tt_block_attn."""
import math

import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle
import synth

from .gpu_cases import DEV, assert_attn_close, np64, say

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def scase(B, S, D, Hq, Hkv, d, lens, seed=0, active=None):
    N = (Hq + 2 * Hkv) * d
    c = dict(B=B, S=S, D=D, Hq=Hq, Hkv=Hkv, d=d, lens=list(lens))
    c["x"] = (synth.normal((B, S, D), 1.0, seed + 1, torch.float32, DEV) +
              synth.normal((B, S, 1), 0.5, seed + 2, torch.float32, DEV)).to(BF16)
    c["shift"] = synth.normal((B, D), 0.1, seed + 3, torch.float32, DEV)
    c["scale"] = synth.normal((B, D), 0.2, seed + 4, torch.float32, DEV)
    c["gate"] = synth.normal((B, D), 1.0, seed + 5, torch.float32, DEV)
    c["w_qkv"] = synth.normal((N, D), 1.0 / math.sqrt(D), seed + 6, BF16, DEV)
    c["w_o"] = synth.normal((D, Hq * d), 1.0 / math.sqrt(Hq * d), seed + 7, BF16, DEV)
    start, ln, total = synth.ragged_context(lens)
    c["kc"] = synth.normal((max(total, 1), Hkv, d), 1.0, seed + 8, BF16, DEV)
    c["vc"] = synth.normal((max(total, 1), Hkv, d), 1.0, seed + 9, BF16, DEV)
    c["ctx_start"], c["ctx_len"] = start.to(DEV), ln.to(DEV)
    c["max_len"] = max(list(lens) + [0])
    c["active"] = None if active is None else torch.tensor(active, dtype=torch.uint8, device=DEV)
    c["shape"] = tt.attn_shape(B, Hq, Hkv, d, S, BF16)
    return c


def chain(c, out=None):
    """ln_modulate -> qkv_proj -> block_attn -> out_proj; returns every stage."""
    B, S, D, Hq, Hkv, d = (c[k] for k in ("B", "S", "D", "Hq", "Hkv", "d"))
    sh = c["shape"]
    h = torch.full((B, S, D), 7.0, dtype=BF16, device=DEV)
    q = torch.full((B, S, Hq, d), 7.0, dtype=BF16, device=DEV)
    k = torch.full((B, S, Hkv, d), 7.0, dtype=BF16, device=DEV)
    v = torch.full((B, S, Hkv, d), 7.0, dtype=BF16, device=DEV)
    o = torch.full((B, S, Hq, d), 7.0, dtype=BF16, device=DEV)
    if out is None:
        out = torch.full((B, S, D), 5.0, dtype=BF16, device=DEV)
    tt.ln_modulate(sh, D, c["x"], c["shift"], c["scale"], h, active=c["active"])
    tt.qkv_proj(sh, D, h, c["w_qkv"], q, k, v, active=c["active"])
    ws = torch.zeros(tt.block_attn_workspace_size(sh, c["max_len"]), dtype=torch.uint8, device=DEV)
    tt.block_attn(sh, q, k, v, c["kc"], c["vc"], c["ctx_start"], c["ctx_len"], c["max_len"], o, ws,
                  active=c["active"])
    tt.out_proj(sh, D, o, c["w_o"], c["gate"], c["x"], out, active=c["active"])
    torch.cuda.synchronize()
    return dict(h=h, q=q, k=k, v=v, o=o, out=out)


def composite(c, out=None):
    D = c["D"]
    if out is None:
        out = torch.full_like(c["x"], 5.0)
    ws = torch.empty(tt.adaln_sublayer_workspace_size(c["shape"], D, c["max_len"]),
                     dtype=torch.uint8, device=DEV)
    tt.adaln_attn_sublayer(c["shape"], D, c["x"], c["shift"], c["scale"], c["gate"], c["w_qkv"],
                           c["w_o"], c["kc"], c["vc"], c["ctx_start"], c["ctx_len"], c["max_len"],
                           out, ws, active=c["active"])
    torch.cuda.synchronize()
    return out


def close(got, want, bound, what):
    g = np64(got) if isinstance(got, torch.Tensor) else got
    err = np.abs(g - want)
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: worst error {worst:.2f} of its bound"


def check_ln(c, h, rows=None):
    """h = LN(x) (1 + scale) + shift: fp32 statistics, one bf16 rounding
    (2^-9 |h|), so 2^-8 |h| plus 1e-5 of the largest |h|."""
    x = np64(c["x"])
    ref = oracle.ln_modulate(x, np64(c["shift"]), np64(c["scale"]))
    sel = slice(None) if rows is None else rows
    close(np64(h)[sel], ref[sel], 2.0 ** -8 * np.abs(ref[sel]) + 1e-5 * np.abs(ref).max(), "ln_modulate")


def proj_bound(a, w, ref):
    """fp32 accumulation of bf16 products then one bf16 rounding: 2^-8 |ref|
    plus 2^-16 of sum_k |a_k w_k| (the accumulation's share, far above its
    sqrt(K) 2^-24 typical size, far below an index mistake's O(1))."""
    return 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * (np.abs(a) @ np.abs(w).T)


def check_qkv(c, st, seqs=None):
    B, S, D, Hq, Hkv, d = (c[k] for k in ("B", "S", "D", "Hq", "Hkv", "d"))
    seqs = list(range(B)) if seqs is None else list(seqs)
    h = np64(st["h"])[seqs].reshape(-1, D)
    w = np64(c["w_qkv"])
    ref = oracle.linear(h, w)
    got = np.concatenate([np64(st["q"])[seqs].reshape(-1, Hq * d), np64(st["k"])[seqs].reshape(-1, Hkv * d),
                          np64(st["v"])[seqs].reshape(-1, Hkv * d)], axis=1)
    close(got, ref, proj_bound(h, w, ref), "qkv_proj")


def check_out(c, st, seqs=None):
    B, S, D, Hq, d = (c[k] for k in ("B", "S", "D", "Hq", "d"))
    seqs = list(range(B)) if seqs is None else list(seqs)
    o = np64(st["o"])[seqs].reshape(len(seqs), S, Hq * d)
    w = np64(c["w_o"])
    x, gate = np64(c["x"])[seqs], np64(c["gate"])[seqs]
    y = oracle.linear(o, w)
    ref = oracle.gate_residual(x, y, gate)
    acc = np.abs(o.reshape(-1, Hq * d)) @ np.abs(w).T
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * np.abs(gate)[:, None, :] * acc.reshape(ref.shape)
    close(np64(st["out"])[seqs], ref, bound, "out_proj")


def check_attn(c, st, seqs=None):
    B = c["B"]
    seqs = list(range(B)) if seqs is None else list(seqs)
    ref, _ = oracle.block_attn(np64(st["q"])[seqs], np64(st["k"])[seqs], np64(st["v"])[seqs],
                               np64(c["kc"]), np64(c["vc"]), np64(c["ctx_start"])[seqs].astype(np.int64),
                               np64(c["ctx_len"])[seqs].astype(np.int64))
    assert_attn_close(np64(st["o"])[seqs], None, ref, None, BF16, "sublayer attention")


CASES = [
    # B, S, D, Hq, Hkv, d, context lengths
    (3, 5, 192, 3, 1, 64, (40, 0, 129)),       # M = 15 (one ragged m-tile), N = 320 (ragged n-tile)
    (40, 5, 64, 2, 1, 64, [7 * i % 50 for i in range(40)]),   # K = 64 (a single step), 2 m-tiles
    (2, 16, 2688, 8, 2, 128, (300, 17)),       # width not a power of two (42 k-steps)
    (8, 16, 512, 4, 2, 128, [64] * 8),         # 8 tiles: the per-XCD tile numbering
    (1, 1, 64, 1, 1, 64, (5,)),                # a single token row (M = 1)
    (2, 64, 128, 2, 1, 128, (10, 300)),        # the longest block (S = 64)
]


@pytest.mark.parametrize("B,S,D,Hq,Hkv,d,lens", CASES)
def test_stages_against_oracle(B, S, D, Hq, Hkv, d, lens):
    say("sublayer stages", dict(B=B, S=S, D=D, Hq=Hq, Hkv=Hkv, d=d))
    c = scase(B, S, D, Hq, Hkv, d, lens, seed=B + D)
    st = chain(c)
    check_ln(c, st["h"])
    check_qkv(c, st)
    check_attn(c, st)
    check_out(c, st)
    got = composite(c)
    assert torch.equal(got, st["out"]), "composite differs from the chain of calls"


def test_in_place_and_inactive():
    c = scase(4, 8, 256, 4, 1, 64, (10, 0, 33, 5), seed=21, active=[1, 0, 1, 1])
    say("sublayer in place / inactive")
    st = chain(c)
    for b in (0, 2, 3):
        check_out(c, st, seqs=[b])
    assert torch.all(st["out"][1] == 5.0) and torch.all(st["h"][1] == 7.0)
    assert torch.all(st["q"][1] == 7.0)
    x0 = c["x"].clone()
    got = composite(c, out=c["x"])                  # out aliases x
    want = st["out"].clone()
    want[1] = x0[1]                                 # inactive rows keep x (untouched)
    assert torch.equal(got, want)


# The sublayer against the oracle end to end from the original inputs (no
# intermediate bytes shared): bf16 roundings of h, q, k, v and o reach the
# output through the projections and the softmax, so the bound is 2^-8 |out|
# plus 3% of the largest |out - x| (the sublayer's own contribution).
def test_end_to_end_against_oracle():
    c = scase(3, 16, 256, 4, 2, 64, (90, 0, 200), seed=31)
    say("sublayer end to end")
    got = composite(c)
    ref = oracle.adaln_attn_sublayer(np64(c["x"]), np64(c["shift"]), np64(c["scale"]),
                                     np64(c["gate"]), np64(c["w_qkv"]), np64(c["w_o"]),
                                     np64(c["kc"]), np64(c["vc"]), np64(c["ctx_start"]).astype(np.int64),
                                     np64(c["ctx_len"]).astype(np.int64), 4, 2, 64)
    delta = np.abs(ref - np64(c["x"])).max()
    close(got, ref, 2.0 ** -8 * np.abs(ref) + 0.03 * delta, "end to end")


# Full size: 64 sequences, S = 16, width 4096, 32 / 2 heads of 128, 1024
# context tokens each (the launch shapes the benchmark times: the QKV
# projection in 256 tiles of 128 x 144, the O projection in 256 of
# 128 x 128).  The QKV projection is checked on every row (an fp64 product
# of 19 GFLOP on the host), the other stages on sampled sequences.
def test_full_size_sampled():
    c = scase(64, 16, 4096, 32, 2, 128, [1024] * 64, seed=41)
    say("sublayer full size")
    st = chain(c)
    seqs = [0, 29, 63]
    check_ln(dict(c, x=c["x"][seqs], shift=c["shift"][seqs], scale=c["scale"][seqs]), st["h"][seqs])
    check_qkv(c, st)
    check_attn(c, st, seqs)
    check_out(c, st, seqs)
    got = composite(c)
    assert torch.equal(got, st["out"])
