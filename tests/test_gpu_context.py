"""GPU parity of the context tower's step over a committed block --
tt_ctx_block_attn (causal attention over [context ; block] with the cache
append) and tt_ctx_advance -- against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle

from .gpu_cases import DEV, assert_attn_close, attn_case, np64, say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _regions(c, room):
    """ctx_end for each sequence: its context plus `room[b]` free tokens.  The
    cases below lay the sequences out with a gap of at least max(room)."""
    st = c["ctx_start"].cpu().numpy()
    return torch.tensor(st + np.asarray(c["lens"]) + np.asarray(room), dtype=torch.int64,
                        device=DEV)


def _run(c, ctx_end=None, max_ctx_len=None, with_lse=True):
    import block_mask_diffusion_tt_amd as tt
    shape = tt.attn_shape(c["B"], c["Hq"], c["Hkv"], c["d"], c["S"], c["dtype"])
    hint = c["max_len"] if max_ctx_len is None else max_ctx_len
    ws = torch.zeros(tt.block_attn_workspace_size(shape, hint), dtype=torch.uint8, device=DEV)
    out = torch.full((c["B"], c["S"], c["Hq"], c["d"]), 7.0, dtype=c["dtype"], device=DEV)
    lse = torch.full((c["B"], c["S"], c["Hq"]), 7.0, dtype=torch.float32, device=DEV) if with_lse else None
    tt.ctx_block_attn(shape, c["q"], c["kb"], c["vb"], c["kc"], c["vc"], c["ctx_start"],
                      c["ctx_len"], hint, out, ws, ctx_end=ctx_end, active=c["active"],
                      residual=c["residual"], lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _np(t):
    return t.detach().cpu().numpy() if t.dtype == torch.float64 else np64(t)


def _oracle(c, seqs=None, kc=None, vc=None):
    """Oracle on the D2H bytes (kc/vc: the cache as it was before the call)."""
    seqs = list(range(c["B"])) if seqs is None else list(seqs)
    starts = c["ctx_start"].cpu().numpy()
    lens = np.asarray(c["lens"])
    kc = c["kc"] if kc is None else kc
    vc = c["vc"] if vc is None else vc
    outs, lses = [], []
    for b in seqs:
        st, n = int(starts[b]), int(lens[b])
        k = np64(kc[st:st + n]) if n else np.zeros((0,) + tuple(kc.shape[1:]))
        v = np64(vc[st:st + n]) if n else np.zeros((0,) + tuple(vc.shape[1:]))
        sel = lambda t: None if t is None else _np(t[b:b + 1])  # noqa: E731
        o, l = oracle.ctx_block_attn(sel(c["q"]), sel(c["kb"]), sel(c["vb"]), k, v,
                                     np.array([0]), np.array([n]), residual=sel(c["residual"]))
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def _check(c, what, seqs=None, **kw):
    say(what, {k: c[k] for k in ("B", "S", "Hq", "Hkv", "d", "dtype")}, "lens", c["lens"][:8])
    out, lse = _run(c, **kw)
    ro, rl = _oracle(c, seqs)
    sl = slice(None) if seqs is None else list(seqs)
    return assert_attn_close(out[sl], lse[sl], ro, rl, c["dtype"], what)


@pytest.mark.parametrize("L", [0, 1, 17, 127, 4096])
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_causal_context_lengths(L, dtype):
    c = attn_case(2, 16, 32, 2, 128, [L, max(L - 1, 0)], dtype=dtype, seed=2000 + L)
    _check(c, f"ctx-tower L={L}")


@pytest.mark.parametrize("S", [1, 4, 16, 64])
@pytest.mark.parametrize("heads", [(4, 1), (8, 8), (32, 2)])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_shapes_bf16(S, heads, d):
    Hq, Hkv = heads
    c = attn_case(3, S, Hq, Hkv, d, [300, 0, 77], dtype=BF16, seed=2100 + S + d + Hq,
                  residual=True, reverse_layout=True, gap=5)
    _check(c, f"ctx-tower S={S} heads={heads} d={d}")


@pytest.mark.parametrize("S,heads,d", [(1, (4, 1), 64), (16, (32, 2), 128), (64, (8, 8), 128)])
def test_causal_shapes_fp32(S, heads, d):
    Hq, Hkv = heads
    c = attn_case(2, S, Hq, Hkv, d, [130, 0], dtype=F32, seed=2200 + S, residual=True)
    _check(c, f"ctx-tower fp32 S={S} heads={heads} d={d}")


# Short contexts with peaked queries: the in-block causal mask decides most of
# the probability mass here, so a wrong mask cannot hide.  The bf16 kernel
# rounds q/sqrt(d)*log2(e) to bf16 for the matrix cores; the oracle gets that
# same rounded query (computed on the host in fp32), and the exact oracle is
# held to the relative-Frobenius bound.
@pytest.mark.parametrize("L", [0, 8, 100])
def test_causal_peaked_short_context(L):
    from .gpu_cases import TOL, peaked_errors, record, rounded_query
    c = attn_case(4, 16, 32, 2, 128, [L, L // 2, 0, L], dtype=BF16, seed=2300 + L, qscale=4.0)
    say("ctx-tower peaked", L)
    out, lse = _run(c)
    qr = rounded_query(c)
    ro, rl = _oracle(dict(c, q=torch.from_numpy(qr)))
    assert_attn_close(out, lse, ro, rl, BF16, f"ctx-tower peaked L={L} (rounded q)")
    eo, _ = _oracle(c)
    e = peaked_errors(out, eo, ro)
    record(f"ctx-tower peaked L={L}", **e)
    assert e["exact_rel_fro"] <= TOL[BF16]["rel_fro"], e


# The cache append: bit-exact copies at the right rows, nothing else written;
# no room or inactive -> untouched; ctx_len unchanged by the attention call;
# tt_ctx_advance then applies the same room rule (bit-exact against the
# oracle's kv_append / ctx_advance).
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_append_and_advance(dtype):
    import block_mask_diffusion_tt_amd as tt
    lens = [40, 0, 513, 64, 7]
    c = attn_case(5, 16, 8, 2, 64, lens, dtype=dtype, seed=2400, gap=32, residual=True,
                  active=[1, 1, 1, 0, 1])
    room = [16, 20, 15, 30, 16]           # sequence 2 has no room, 3 is inactive
    ctx_end = _regions(c, room)
    kc0, vc0 = c["kc"].clone(), c["vc"].clone()
    len0 = c["ctx_len"].clone()
    say("append", dtype)
    out, lse = _run(c, ctx_end=ctx_end)
    ro, rl = _oracle(c, [0, 1, 2, 4], kc=kc0, vc=vc0)
    assert_attn_close(out[[0, 1, 2, 4]], lse[[0, 1, 2, 4]], ro, rl, dtype, "append call attention")
    assert torch.all(out[3] == 7.0)                       # inactive: not written
    assert torch.equal(c["ctx_len"], len0)
    st = c["ctx_start"].cpu().numpy()
    f32 = lambda t: t.cpu().float().numpy()  # noqa: E731  (exact for bf16 and fp32)
    ek, ev, app = oracle.kv_append(f32(kc0), f32(vc0), f32(c["kb"]), f32(c["vb"]), st,
                                   ctx_end.cpu().numpy(), len0.cpu().numpy(),
                                   c["active"].cpu().numpy())
    assert app.tolist() == [True, True, False, False, True]
    assert np.array_equal(f32(c["kc"]), ek)
    assert np.array_equal(f32(c["vc"]), ev)
    appended = torch.full((5,), 9, dtype=torch.uint8, device=DEV)
    tt.ctx_advance(5, 16, c["ctx_start"], ctx_end, c["ctx_len"], active=c["active"],
                   appended=appended)
    torch.cuda.synchronize()
    n2, app2 = oracle.ctx_advance(16, st, ctx_end.cpu().numpy(), len0.cpu().numpy(),
                                  c["active"].cpu().numpy())
    assert c["ctx_len"].cpu().tolist() == n2.tolist()
    assert appended.cpu().tolist() == [int(x) for x in app2]


# Two blocks in a row through the library only: the context tower commits
# block A (attention + append on every layer of a 2-layer cache, then one
# advance), then the denoiser attends block B over the grown cache; both
# against the oracle on the explicit concatenation.
def test_commit_then_denoise_next_block():
    import block_mask_diffusion_tt_amd as tt
    import synth
    B, S, Hq, Hkv, d, layers = 3, 16, 32, 2, 128, 2
    lens = [1000, 0, 333]
    cap = [l + 2 * S for l in lens]
    starts = np.concatenate([[0], np.cumsum(cap)[:-1]])
    T = int(sum(cap))
    ctx_start = torch.tensor(starts, dtype=torch.int64, device=DEV)
    ctx_end = torch.tensor(starts + np.asarray(cap), dtype=torch.int64, device=DEV)
    ctx_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    shape = tt.attn_shape(B, Hq, Hkv, d, S, BF16)
    ws = torch.zeros(tt.block_attn_workspace_size(shape, max(cap)), dtype=torch.uint8, device=DEV)
    kc = [synth.normal((T, Hkv, d), 1.0, 2500 + l, BF16, DEV) for l in range(layers)]
    vc = [synth.normal((T, Hkv, d), 1.0, 2510 + l, BF16, DEV) for l in range(layers)]
    kc0 = [x.clone() for x in kc]
    vc0 = [x.clone() for x in vc]
    blk = [[synth.normal(shp, 1.0, 2520 + 10 * l + i, BF16, DEV)
            for i, shp in enumerate([(B, S, Hq, d), (B, S, Hkv, d), (B, S, Hkv, d)])]
           for l in range(layers)]
    say("commit block A on", layers, "layers")
    for l in range(layers):
        out = torch.empty((B, S, Hq, d), dtype=BF16, device=DEV)
        q, kb, vb = blk[l]
        tt.ctx_block_attn(shape, q, kb, vb, kc[l], vc[l], ctx_start, ctx_len, max(lens), out, ws,
                          ctx_end=ctx_end)
        torch.cuda.synchronize()
        for b in range(B):
            st, n = int(starts[b]), lens[b]
            ro, _ = oracle.ctx_block_attn(np64(q[b:b + 1]), np64(kb[b:b + 1]), np64(vb[b:b + 1]),
                                          np64(kc0[l][st:st + n]), np64(vc0[l][st:st + n]),
                                          np.array([0]), np.array([n]))
            assert_attn_close(out[b:b + 1], None, ro, None, BF16, f"commit layer {l} seq {b}")
    tt.ctx_advance(B, S, ctx_start, ctx_end, ctx_len)
    torch.cuda.synchronize()
    assert ctx_len.cpu().tolist() == [l + S for l in lens]
    say("denoise block B over the grown cache")
    q2 = synth.normal((B, S, Hq, d), 1.0, 2590, BF16, DEV)
    k2 = synth.normal((B, S, Hkv, d), 1.0, 2591, BF16, DEV)
    v2 = synth.normal((B, S, Hkv, d), 1.0, 2592, BF16, DEV)
    for l in range(layers):
        out = torch.empty((B, S, Hq, d), dtype=BF16, device=DEV)
        tt.block_attn(shape, q2, k2, v2, kc[l], vc[l], ctx_start, ctx_len, max(cap), out, ws)
        torch.cuda.synchronize()
        for b in range(B):
            st, n = int(starts[b]), lens[b]
            kcat = np.concatenate([np64(kc0[l][st:st + n]), np64(blk[l][1][b])], axis=0)
            vcat = np.concatenate([np64(vc0[l][st:st + n]), np64(blk[l][2][b])], axis=0)
            ro, _ = oracle.block_attn(np64(q2[b:b + 1]), np64(k2[b:b + 1]), np64(v2[b:b + 1]),
                                      kcat, vcat, np.array([0]), np.array([n + S]))
            assert_attn_close(out[b:b + 1], None, ro, None, BF16, f"next block layer {l} seq {b}")


# Full size, the launch the benchmark times: batch 64, context 8192, S = 16,
# append on -- sampled sequences against the oracle, every appended row
# checked bit-exactly.
def test_headline_ctx_commit_sampled():
    c = attn_case(64, 16, 32, 2, 128, [8192] * 64, dtype=BF16, seed=2600, gap=16)
    ctx_end = _regions(c, [16] * 64)
    kc0, vc0 = c["kc"].clone(), c["vc"].clone()
    say("headline ctx-tower 64x8192")
    out, lse = _run(c, ctx_end=ctx_end)
    seqs = [0, 31, 63]
    ro, rl = _oracle(c, seqs, kc=kc0, vc=vc0)
    assert_attn_close(out[seqs], lse[seqs], ro, rl, BF16, "headline ctx-tower")
    st = c["ctx_start"].cpu()
    for b in range(64):
        a = int(st[b]) + 8192
        assert torch.equal(c["kc"][a:a + 16], c["kb"][b]) and torch.equal(c["vc"][a:a + 16], c["vb"][b])
    keep = torch.ones(c["kc"].shape[0], dtype=torch.bool)
    for b in range(64):
        a = int(st[b]) + 8192
        keep[a:a + 16] = False
    assert torch.equal(c["kc"][keep.to(DEV)], kc0[keep.to(DEV)])


def test_ctx_deterministic_and_chunking():
    c = attn_case(2, 16, 32, 2, 128, [3000, 1500], dtype=BF16, seed=2700)
    a, la = _run(c)
    b, lb = _run(c)
    assert torch.equal(a, b) and torch.equal(la, lb)
    h, lh = _run(c, max_ctx_len=64)
    ro, rl = _oracle(c)
    assert_attn_close(h, lh, ro, rl, BF16, "ctx-tower hint = 64")
