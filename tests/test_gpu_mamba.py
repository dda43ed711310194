"""GPU parity of tt_mamba_block_scan (one Mamba-2 layer's mixer over a block,
seeded with the context tower's conv/SSM states) against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle.mamba as mb
import synth

from .gpu_cases import DEV, np64, say

pytestmark = pytest.mark.gpu
BF16, F32 = torch.bfloat16, torch.float32


def mcase(B, S, H, P, N, G, W=4, dtype=BF16, seed=0, active=None):
    C = H * P + 2 * G * N
    f = lambda shape, std, k: synth.normal(shape, std, seed + k, torch.float32, DEV)  # noqa: E731
    c = dict(B=B, S=S, H=H, P=P, N=N, G=G, W=W, dtype=dtype)
    c["xbc"] = synth.normal((B, S, C), 1.0, seed + 1, dtype, DEV)
    c["dt_raw"] = f((B, S, H), 1.0, 2) - 1.0
    c["conv_state"] = synth.normal((B, C, W - 1), 1.0, seed + 3, dtype, DEV)
    c["ssm_state"] = f((B, H, P, N), 1.0, 4)
    c["conv_w"] = f((C, W), 0.5, 5)
    c["conv_b"] = f((C,), 0.1, 6)
    c["A_log"] = torch.log(torch.linspace(1.0, 16.0, H, device=DEV))
    c["dt_bias"] = f((H,), 0.3, 7)
    c["D"] = f((H,), 1.0, 8)
    c["active"] = None if active is None else torch.tensor(active, dtype=torch.uint8, device=DEV)
    return c


def run(c, states_out=False, in_place=True):
    shape = tt.mamba_shape(c["B"], c["H"], c["P"], c["N"], c["G"], c["W"], c["S"], c["dtype"])
    y = torch.full((c["B"], c["S"], c["H"] * c["P"]), 7.0, dtype=c["dtype"], device=DEV)
    cso = sso = None
    if states_out:
        cso = torch.full_like(c["conv_state"], 5.0)
        sso = c["ssm_state"] if in_place else torch.full_like(c["ssm_state"], 5.0)
    ws = torch.empty(tt.mamba_workspace_size(shape), dtype=torch.uint8, device=DEV)
    tt.mamba_block_scan(shape, c["xbc"], c["dt_raw"], c["conv_state"], c["ssm_state"], c["conv_w"],
                        c["A_log"], y, ws, conv_b=c["conv_b"], dt_bias=c["dt_bias"], D=c["D"],
                        active=c["active"], conv_state_out=cso, ssm_state_out=sso)
    torch.cuda.synchronize()
    return y, cso, sso


def ref(c, seqs=None, ssm_state=None, return_state=False):
    seqs = list(range(c["B"])) if seqs is None else list(seqs)
    ss = c["ssm_state"] if ssm_state is None else ssm_state
    return mb.mamba_block_scan(np64(c["xbc"][seqs]), np64(c["dt_raw"][seqs]),
                               np64(c["conv_state"][seqs]), np64(ss[seqs]), np64(c["conv_w"]),
                               np64(c["conv_b"]), np64(c["A_log"]), np64(c["dt_bias"]),
                               np64(c["D"]), c["G"], c["N"], c["P"], return_state=return_state)


def close(got, want, dtype, what):
    """fp32 arithmetic throughout; a bf16 output adds half an ulp (2^-9
    relative), so the bound is 2^-8 |ref| plus 1e-5 of the largest |ref| for
    bf16, 1e-5 of the largest |ref| for fp32."""
    g = np64(got) if isinstance(got, torch.Tensor) else got
    w = np.asarray(want).reshape(g.shape)
    scale = float(np.abs(w).max())
    rel = 2.0 ** -8 if dtype == BF16 else 0.0
    bound = rel * np.abs(w) + 1e-5 * scale
    err = np.abs(g - w)
    assert np.all(err <= bound), f"{what}: worst {float((err / bound).max()):.2f} of the bound"


@pytest.mark.parametrize("P,N", [(64, 128), (64, 64), (32, 128), (32, 64)])
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_shapes(P, N, dtype):
    c = mcase(2, 16, 4, P, N, 2, dtype=dtype, seed=10 + P + N)
    say("mamba", {k: c[k] for k in ("B", "S", "H", "P", "N", "G", "W", "dtype")})
    y, _, _ = run(c)
    close(y, ref(c), dtype, f"P={P} N={N}")


@pytest.mark.parametrize("S,W,G", [(1, 4, 1), (4, 2, 2), (5, 3, 4), (64, 4, 8)])
def test_block_lengths_and_conv_widths(S, W, G):
    c = mcase(2, S, 8, 64, 128, G, W=W, seed=30 + S + W)
    say("mamba S W G", S, W, G)
    y, _, _ = run(c)
    close(y, ref(c), BF16, f"S={S} W={W} G={G}")


# The context tower taking a committed block: the final SSM state in place,
# the conv state to a second buffer, against the oracle's final states.
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_state_update(dtype):
    c = mcase(3, 16, 8, 64, 128, 2, dtype=dtype, seed=50)
    y_ref, conv_ref, ssm_ref = ref(c, return_state=True)
    y, cso, sso = run(c, states_out=True, in_place=True)
    close(y, y_ref, dtype, "state update y")
    np.testing.assert_array_equal(np64(cso), conv_ref)          # raw inputs, exact
    close(sso, ssm_ref, F32, "final SSM state")


# Seeding end to end on the GPU: the context (16 tokens from zero states)
# through the library with its state outputs, then the next block seeded
# with them, equals one oracle scan over the 32 tokens from zero states.
def test_seeding_composition():
    B, S, H, P, N, G, W = 2, 16, 4, 64, 128, 2, 4
    ctx = mcase(B, S, H, P, N, G, W=W, dtype=F32, seed=60)
    ctx["conv_state"] = torch.zeros_like(ctx["conv_state"])
    ctx["ssm_state"] = torch.zeros_like(ctx["ssm_state"])
    _, cso, sso = run(ctx, states_out=True, in_place=False)
    blk = dict(ctx)
    blk["xbc"] = synth.normal(ctx["xbc"].shape, 1.0, 61, F32, DEV)
    blk["dt_raw"] = synth.normal(ctx["dt_raw"].shape, 1.0, 62, F32, DEV) - 1.0
    blk["conv_state"], blk["ssm_state"] = cso, sso
    y, _, _ = run(blk)
    full = mb.mamba_block_scan(
        np.concatenate([np64(ctx["xbc"]), np64(blk["xbc"])], axis=1),
        np.concatenate([np64(ctx["dt_raw"]), np64(blk["dt_raw"])], axis=1),
        np.zeros((B, H * P + 2 * G * N, W - 1)), np.zeros((B, H, P, N)), np64(ctx["conv_w"]),
        np64(ctx["conv_b"]), np64(ctx["A_log"]), np64(ctx["dt_bias"]), np64(ctx["D"]), G, N, P)
    close(y, full[:, S:], F32, "seeded block vs one scan of the concatenation")


def test_inactive_untouched():
    c = mcase(3, 8, 4, 32, 64, 2, seed=70, active=[1, 0, 1])
    y, cso, sso = run(c, states_out=True, in_place=False)
    close(y[[0, 2]], ref(c, [0, 2]), BF16, "active")
    assert torch.all(y[1] == 7.0) and torch.all(cso[1] == 5.0) and torch.all(sso[1] == 5.0)


def test_deterministic():
    c = mcase(2, 16, 8, 64, 128, 2, seed=80)
    a, _, _ = run(c)
    b, _, _ = run(c)
    assert torch.equal(a, b)


# Full size: 64 sequences, S = 16, 64 heads of 64 channels, d_state 128, 8
# groups, conv width 4 (the launch the benchmark times) -- sampled sequences.
def test_full_size_sampled():
    c = mcase(64, 16, 64, 64, 128, 8, seed=90)
    say("mamba full size")
    y, _, _ = run(c)
    seqs = [0, 33, 63]
    close(y[seqs], ref(c, seqs), BF16, "full size")


def _mshapes(seed, n):
    """Seeded shapes: the four (P, N) pairs in turn (N = 2P takes the
    one-launch form for S <= 16), S on both sides of 16, head counts whose
    sequence x head units leave the XCD-aware grid partly idle, every conv
    width, both dtypes, and the final states on every other case."""
    rng = np.random.default_rng(seed)
    pn = [(64, 128), (32, 64), (64, 64), (32, 128)]
    out = []
    for i in range(n):
        P, N = pn[i % 4]
        S = int(rng.integers(1, 17)) if i < n - 2 else int(rng.integers(17, 65))
        H = int(rng.choice([4, 8, 12]))
        G = int(rng.choice([g for g in (1, 2, 4) if H % g == 0]))
        out.append((int(rng.integers(1, 6)), S, H, P, N, G, int(rng.integers(2, 5)),
                    BF16 if rng.random() < 0.6 else F32, bool(i % 2)))
    return out


@pytest.mark.parametrize("B,S,H,P,N,G,W,dtype,states", _mshapes(2026, 8))
def test_random_shapes(B, S, H, P, N, G, W, dtype, states):
    c = mcase(B, S, H, P, N, G, W=W, dtype=dtype, seed=100 + B * 97 + S * 13 + H + W)
    say("mamba random", B, S, H, P, N, G, W, dtype, "states" if states else "")
    if states:
        y_ref, conv_ref, ssm_ref = ref(c, return_state=True)
        y, cso, sso = run(c, states_out=True, in_place=False)
        np.testing.assert_array_equal(np64(cso), conv_ref)
        close(sso, ssm_ref, F32, "random final SSM state")
    else:
        y_ref = ref(c)
        y, _, _ = run(c)
    close(y, y_ref, dtype, f"random B={B} S={S} H={H} P={P} N={N} G={G} W={W}")
