"""Input builders and comparison helpers for the GPU parity tests.

Inputs come from the seeded generators in `synth`; the oracle always gets
D2H copies of exactly the bytes the GPU consumed (widened exactly to fp64).
"""
import sys

import numpy as np
import torch

import synth

DEV = "cuda"

# Tolerances: the contract's max-abs bounds, plus relative-Frobenius and lse
# bounds because N(0,1) inputs make outputs small (near-uniform attention).
TOL = {torch.bfloat16: dict(max_abs=2e-2, rel_fro=1e-2, lse=2e-2),
       torch.float32: dict(max_abs=1e-5, rel_fro=1e-5, lse=1e-5)}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def record(what, **values):
    """Prints a measured quantity of a test and, when TT_TEST_RECORD names a
    file, appends it there as one JSON line (for numbers that are reported
    rather than asserted, such as the peaked cases' exact-oracle error)."""
    import json
    import os
    say(what, values)
    path = os.environ.get("TT_TEST_RECORD")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(dict(what=what, **values)) + "\n")


def peaked_errors(out, eo, ro_rounded_q):
    """Max-abs errors of a peaked case: the kernel against the exact oracle,
    and how far the operand rounding of q' alone moves the exact result (the
    oracle on the rounded query against the exact oracle)."""
    o = np64(out) if isinstance(out, torch.Tensor) else out
    return dict(exact_max_abs=float(np.abs(o - eo).max()),
                rounding_shift_max_abs=float(np.abs(ro_rounded_q - eo).max()),
                exact_rel_fro=float(np.linalg.norm(o - eo) / np.linalg.norm(eo)))


def np64(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def attn_case(B, S, Hq, Hkv, d, lens, dtype=torch.bfloat16, seed=0, qscale=1.0, ada=False,
              residual=False, reverse_layout=False, gap=0, active=None, ada_std=(0.1, 0.2, 1.0)):
    """One attention layer's inputs.  Sequences' context tokens live in one
    cache, back to back (or in reverse order, with `gap` unused tokens between
    them, to exercise ctx_start)."""
    lens = [int(x) for x in lens]
    order = list(range(B))[::-1] if reverse_layout else list(range(B))
    starts = [0] * B
    pos = 0
    for b in order:
        starts[b] = pos
        pos += lens[b] + gap
    total = max(pos, 1)
    c = dict(B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, lens=lens, max_len=max(lens + [0]))
    c["q"] = synth.normal((B, S, Hq, d), qscale, seed + 1, dtype, DEV)
    c["kb"] = synth.normal((B, S, Hkv, d), 1.0, seed + 2, dtype, DEV)
    c["vb"] = synth.normal((B, S, Hkv, d), 1.0, seed + 3, dtype, DEV)
    c["kc"] = synth.normal((total, Hkv, d), 1.0, seed + 4, dtype, DEV)
    c["vc"] = synth.normal((total, Hkv, d), 1.0, seed + 5, dtype, DEV)
    c["ctx_start"] = torch.tensor(starts, dtype=torch.int64, device=DEV)
    c["ctx_len"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    W = Hq * d
    if ada:
        c["shift"] = synth.normal((B, W), ada_std[0], seed + 6, torch.float32, DEV)
        c["scale"] = synth.normal((B, W), ada_std[1], seed + 7, torch.float32, DEV)
        c["gate"] = synth.normal((B, W), ada_std[2], seed + 8, torch.float32, DEV)
    else:
        c["shift"] = c["scale"] = c["gate"] = None
    c["residual"] = synth.normal((B, S, Hq, d), 1.0, seed + 9, dtype, DEV) if residual else None
    c["active"] = None if active is None else torch.tensor(active, dtype=torch.uint8, device=DEV)
    return c


def run_attn(c, max_ctx_len=None, out=None, with_lse=True):
    import block_mask_diffusion_tt_amd as tt
    shape = tt.attn_shape(c["B"], c["Hq"], c["Hkv"], c["d"], c["S"], c["dtype"])
    hint = c["max_len"] if max_ctx_len is None else max_ctx_len
    ws = torch.zeros(tt.block_attn_workspace_size(shape, hint), dtype=torch.uint8, device=DEV)
    if out is None:
        out = torch.full((c["B"], c["S"], c["Hq"], c["d"]), 7.0, dtype=c["dtype"], device=DEV)
    lse = torch.full((c["B"], c["S"], c["Hq"]), 7.0, dtype=torch.float32, device=DEV) if with_lse else None
    tt.block_attn(shape, c["q"], c["kb"], c["vb"], c["kc"], c["vc"], c["ctx_start"], c["ctx_len"],
                  hint, out, ws, active=c["active"], ada_shift=c["shift"], ada_scale=c["scale"],
                  ada_gate=c["gate"], residual=c["residual"], lse=lse)
    torch.cuda.synchronize()
    return out, lse


def rounded_query(c):
    """The bf16 path's documented operand rounding of the modulated query:
    q' = q * (1 + scale) + shift in fp32, times log2(e)/sqrt(d) (fp32), rounded
    to bf16 (nearest-even), returned in fp64 divided by that same factor -- so
    the oracle fed with it and no modulation evaluates attention of exactly
    the query the matrix cores see."""
    q = c["q"].detach().float().cpu()
    B, S, Hq, d = q.shape
    if c["scale"] is not None:
        q = q * (1.0 + c["scale"].detach().cpu().reshape(B, 1, Hq, d))
    if c["shift"] is not None:
        q = q + c["shift"].detach().cpu().reshape(B, 1, Hq, d)
    f = torch.tensor(1.4426950408889634, dtype=torch.float32) / torch.sqrt(torch.tensor(float(d), dtype=torch.float32))
    qb = (q * f).to(torch.bfloat16).to(torch.float64)
    return (qb / f.double()).numpy()


def oracle_attn(c, seqs=None, rounded_q=False):
    """Oracle on the D2H bytes; `seqs` restricts to a subset of sequences
    (sampled checks at full size).  Returns (out, lse) for those sequences.
    With rounded_q the oracle gets rounded_query(c) and no shift/scale."""
    import oracle
    seqs = list(range(c["B"])) if seqs is None else list(seqs)
    qr = rounded_query(c) if rounded_q else None
    starts = c["ctx_start"].cpu().numpy()
    lens = c["ctx_len"].cpu().numpy()
    kc_all, vc_all = c["kc"], c["vc"]
    outs, lses = [], []
    for b in seqs:
        st, n = int(starts[b]), int(lens[b])
        kc = np64(kc_all[st:st + n]) if n else np.zeros((0,) + tuple(kc_all.shape[1:]))
        vc = np64(vc_all[st:st + n]) if n else np.zeros((0,) + tuple(vc_all.shape[1:]))
        sel = lambda t: None if t is None else np64(t[b:b + 1])  # noqa: E731
        if rounded_q:
            o, l = oracle.block_attn(qr[b:b + 1], sel(c["kb"]), sel(c["vb"]), kc, vc,
                                     np.array([0]), np.array([n]), gate=sel(c["gate"]),
                                     residual=sel(c["residual"]))
        else:
            o, l = oracle.block_attn(sel(c["q"]), sel(c["kb"]), sel(c["vb"]), kc, vc,
                                     np.array([0]), np.array([n]), shift=sel(c["shift"]),
                                     scale=sel(c["scale"]), gate=sel(c["gate"]),
                                     residual=sel(c["residual"]))
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def assert_attn_close(out, lse, ref_out, ref_lse, dtype, what="", gate=None):
    """Elementwise bound: the contract's max-abs error applies to the
    attention output o; out = residual + gate * o multiplies that error by
    |gate| and the store rounds once more (half an ulp of |out|: 2^-9 |out| in
    bf16, 2^-24 |out| in fp32; 2^-8 / 2^-23 allow for the fp32 epilogue)."""
    tol = TOL[dtype]
    o = np64(out) if isinstance(out, torch.Tensor) else out
    err = np.abs(o - ref_out)
    g = 1.0
    if gate is not None:
        gv = np64(gate) if isinstance(gate, torch.Tensor) else gate
        B, S, Hq, d = ref_out.shape
        g = np.maximum(1.0, np.abs(gv.reshape(B, 1, Hq, d)))
    rel = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -23
    bound = tol["max_abs"] * g + rel * np.abs(ref_out)
    worst = float((err / bound).max()) if err.size else 0.0
    max_abs = float(err.max()) if err.size else 0.0
    fro = float(np.linalg.norm(o - ref_out) / max(np.linalg.norm(ref_out), 1e-30))
    assert worst <= 1.0, f"{what}: error {max_abs:.3e} exceeds its bound (ratio {worst:.2f})"
    assert fro <= tol["rel_fro"], f"{what}: rel fro {fro:.3e} > {tol['rel_fro']}"
    if lse is not None:
        le = np.abs((np64(lse) if isinstance(lse, torch.Tensor) else lse) - ref_lse)
        assert float(le.max()) <= tol["lse"], f"{what}: lse err {float(le.max()):.3e}"
    return max_abs, fro
