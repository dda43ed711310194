"""GPU parity of tt_block_attn against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from .gpu_cases import (TOL, assert_attn_close, attn_case, np64, oracle_attn, peaked_errors,
                        record, run_attn, say)

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _check(c, what, seqs=None, **kw):
    say(what, {k: c[k] for k in ("B", "S", "Hq", "Hkv", "d", "dtype")}, "lens", c["lens"][:8])
    out, lse = run_attn(c, **kw)
    ro, rl = oracle_attn(c, seqs)
    sl = slice(None) if seqs is None else list(seqs)
    gate = None if c["gate"] is None else c["gate"][sl]
    return assert_attn_close(out[sl], lse[sl], ro, rl, c["dtype"], what, gate=gate)


# The tiny fp32 step: batch 1, 4 query heads / 1 KV head, d = 64, 128 context
# tokens, S = 16, Q/K/V ~ N(0, 1).
def test_tiny_fp32_step():
    c = attn_case(1, 16, 4, 1, 64, [128], dtype=F32, seed=1)
    _check(c, "tiny fp32")


@pytest.mark.parametrize("L", [0, 1, 15, 16, 17, 127, 4096])
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_context_lengths(L, dtype):
    c = attn_case(2, 16, 32, 2, 128, [L, max(L - 1, 0)], dtype=dtype, seed=10 + L)
    _check(c, f"L={L}")


@pytest.mark.parametrize("S", [1, 4, 16, 64])
@pytest.mark.parametrize("heads", [(4, 1), (8, 8), (32, 2)])
@pytest.mark.parametrize("d", [64, 128])
def test_shapes_bf16(S, heads, d):
    Hq, Hkv = heads
    c = attn_case(3, S, Hq, Hkv, d, [300, 0, 77], dtype=BF16, seed=100 + S + d + Hq,
                  ada=True, residual=True, reverse_layout=True, gap=5)
    _check(c, f"S={S} heads={heads} d={d}")


@pytest.mark.parametrize("S,heads,d", [(1, (4, 1), 64), (16, (32, 2), 128), (64, (8, 8), 128),
                                       (4, (32, 2), 64)])
def test_shapes_fp32(S, heads, d):
    Hq, Hkv = heads
    c = attn_case(2, S, Hq, Hkv, d, [130, 33], dtype=F32, seed=200 + S, ada=True, residual=True)
    _check(c, f"fp32 S={S} heads={heads} d={d}")


# Peaked attention (q x 4) and short contexts, where the block keys carry a
# large share of the mass: a wrong block-local part cannot hide here.  The
# bf16 path rounds the modulated query to bf16 for the matrix cores (its
# documented operand precision); with q x 4 that rounding alone moves scores
# by up to ~0.03 log2 units, so the max-abs bound is applied against the
# oracle evaluated on that rounded query, and the exact oracle is held to the
# relative-Frobenius bound.  The max-abs error against the exact oracle is
# reported (printed, and recorded when TT_TEST_RECORD is set) next to the
# shift that the rounding of q' alone causes.
def _check_peaked(c, what):
    say(what, {k: c[k] for k in ("B", "S", "Hq", "Hkv", "d", "dtype")}, "lens", c["lens"])
    out, lse = run_attn(c)
    ro, rl = oracle_attn(c, rounded_q=True)
    assert_attn_close(out, lse, ro, rl, BF16, what + " (rounded q')", gate=c["gate"])
    eo, _ = oracle_attn(c)
    e = peaked_errors(out, eo, ro)
    record(what, **e)
    assert e["exact_rel_fro"] <= TOL[BF16]["rel_fro"], f"{what}: rel fro vs exact {e}"
    return out


@pytest.mark.parametrize("L", [8, 64, 128, 2048])
def test_peaked_small_context(L):
    c = attn_case(4, 16, 32, 2, 128, [L, L // 2, 0, L], dtype=BF16, seed=300 + L, qscale=4.0,
                  ada=True)
    c["gate"] = None
    out = _check_peaked(c, f"peaked L={L}")
    assert float(np.sqrt((np64(out) ** 2).mean())) > 0.2    # outputs are not near zero


@pytest.mark.parametrize("L", [8, 128])
def test_peaked_gated(L):
    c = attn_case(4, 16, 32, 2, 128, [L, L // 2, 0, L], dtype=BF16, seed=350 + L, qscale=4.0,
                  ada=True, residual=True)
    _check_peaked(c, f"peaked gated L={L}")


# Moderately peaked (q x 2) against the exact oracle with the plain bound.
def test_q_x2_exact_bound():
    c = attn_case(4, 16, 32, 2, 128, [64, 700, 0, 2048], dtype=BF16, seed=390, qscale=2.0,
                  ada=True)
    c["gate"] = None
    _check(c, "q x 2 exact")


# One workspace serves calls of different shapes in a row.
def test_workspace_reuse_across_shapes():
    import block_mask_diffusion_tt_amd as tt
    big = attn_case(4, 16, 32, 2, 128, [3000, 100, 2500, 64], dtype=BF16, seed=395, ada=True)
    small = attn_case(2, 4, 8, 2, 64, [900, 1200], dtype=BF16, seed=396)
    ref_big, _ = run_attn(big)
    ref_small, _ = run_attn(small)
    shapes = [tt.attn_shape(x["B"], x["Hq"], x["Hkv"], x["d"], x["S"], BF16) for x in (big, small)]
    n = max(tt.block_attn_workspace_size(sh, x["max_len"]) for sh, x in zip(shapes, (big, small)))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for x, sh, ref in [(big, shapes[0], ref_big), (small, shapes[1], ref_small),
                       (big, shapes[0], ref_big), (big, shapes[0], ref_big),
                       (small, shapes[1], ref_small)]:
        out = torch.empty_like(ref)
        tt.block_attn(sh, x["q"], x["kb"], x["vb"], x["kc"], x["vc"], x["ctx_start"], x["ctx_len"],
                      x["max_len"], out, ws, ada_shift=x["shift"], ada_scale=x["scale"],
                      ada_gate=x["gate"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_inactive_sequences_untouched():
    c = attn_case(3, 16, 8, 2, 64, [50, 60, 70], dtype=BF16, seed=400, active=[1, 0, 1])
    out, lse = run_attn(c)
    ro, rl = oracle_attn(c, [0, 2])
    assert_attn_close(out[[0, 2]], lse[[0, 2]], ro, rl, BF16, "active rows", gate=None)
    assert torch.all(out[1] == 7.0) and torch.all(lse[1] == 7.0)


def test_residual_aliases_out():
    c = attn_case(2, 16, 32, 2, 128, [200, 90], dtype=BF16, seed=500, ada=True, residual=True)
    ro, rl = oracle_attn(c)
    buf = c["residual"].clone()
    c["residual"] = buf
    out, lse = run_attn(c, out=buf)
    assert out.data_ptr() == buf.data_ptr()
    assert_attn_close(out, lse, ro, rl, BF16, "aliased residual", gate=c["gate"])


# P10: the split of the context into chunks does not change the result beyond
# rounding; a launch-size hint smaller than the real length stays correct.
def test_chunking_invariance_and_small_hint():
    c = attn_case(2, 16, 32, 2, 128, [3000, 1500], dtype=BF16, seed=600, ada=True)
    a, la = run_attn(c)
    b, lb = run_attn(c, max_ctx_len=64)
    ro, rl = oracle_attn(c)
    assert_attn_close(a, la, ro, rl, BF16, "hint = max len", gate=c["gate"])
    assert_attn_close(b, lb, ro, rl, BF16, "hint = 64", gate=c["gate"])


def test_deterministic():
    c = attn_case(4, 16, 32, 2, 128, [2048, 999, 1, 4000], dtype=BF16, seed=700, ada=True)
    a, la = run_attn(c)
    b, lb = run_attn(c)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_empty_batch():
    c = attn_case(1, 16, 32, 2, 128, [10], dtype=BF16, seed=800)
    import block_mask_diffusion_tt_amd as tt
    shape = tt.attn_shape(0, 32, 2, 128, 16, BF16)
    tt.block_attn(shape, c["q"], c["kb"], c["vb"], c["kc"], c["vc"], c["ctx_start"],
                  c["ctx_len"], 0, c["q"], None)


# Single sequence, bf16, 32/2 heads, d = 128, 4096 context tokens, S = 16,
# adaLN vectors present (the second workload of the method's configurations).
def test_single_sequence_4096():
    c = attn_case(1, 16, 32, 2, 128, [4096], dtype=BF16, seed=900, ada=True)
    _check(c, "single seq 4096")


# Ragged batch 64, contexts uniform in [1024, 8192] (full size, the launch the
# benchmark times) -- checked on a sample of sequences.
def test_ragged_batch64_sampled():
    import synth
    lens = synth.uniform_int(64, 1024, 8192, seed=3).tolist()
    c = attn_case(64, 16, 32, 2, 128, lens, dtype=BF16, seed=1000, ada=True)
    _check(c, "ragged 64", seqs=[0, 17, 40, 63])


# Value magnitudes far from 1: the bf16 path stores each unit's normalised
# output in fp16 with a power-of-two row scale, which must neither overflow
# (|V| beyond the fp16 range) nor lose relative precision (|V| far below it).
# Scaling V by a power of two is exact in bf16; the relative Frobenius check
# is the meaningful one for the tiny case.
# The output (no residual) is linear in V, so both sides are divided by the
# scale and held to the unit-scale bound.
@pytest.mark.parametrize("vscale", [2.0 ** 17, 2.0 ** -20])
def test_value_magnitudes(vscale):
    c = attn_case(3, 16, 32, 2, 128, [5000, 700, 0], dtype=BF16, seed=1400, ada=True)
    for key in ("vb", "vc"):
        c[key].mul_(vscale)
    what = f"|V| scaled by {vscale:g}"
    say(what)
    out, lse = run_attn(c)
    ro, rl = oracle_attn(c)
    assert np.isfinite(np64(out)).all(), what
    assert_attn_close(np64(out) / vscale, lse, ro / vscale, rl, BF16, what, gate=c["gate"])


# Throughput shape: batch 128, contexts uniform in [2048, 16384] (full size,
# about 1.2 M context tokens) -- sampled, including the shortest and longest
# sequences of the draw.
def test_throughput_batch128_sampled():
    import synth
    lens = synth.uniform_int(128, 2048, 16384, seed=5).tolist()
    picks = sorted({0, 127, int(np.argmin(lens)), int(np.argmax(lens))})
    c = attn_case(128, 16, 32, 2, 128, lens, dtype=BF16, seed=1300, ada=True)
    _check(c, "throughput 128", seqs=picks)


def test_headline_batch64_ctx8192_sampled():
    c = attn_case(64, 16, 32, 2, 128, [8192] * 64, dtype=BF16, seed=1100, ada=True)
    _check(c, "headline 64x8192", seqs=[0, 31, 63])


# Block-size sweep shape: batch 8, context 32768, S in {4, 16, 64} (sampled)
@pytest.mark.parametrize("S", [4, 16, 64])
def test_context_32768_sampled(S):
    c = attn_case(8, S, 32, 2, 128, [32768] * 8, dtype=BF16, seed=1200 + S)
    _check(c, f"ctx 32768 S={S}", seqs=[0, 7])


def _many_chunk_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(0, 9217, size=B)]
        lens[int(rng.integers(0, B))] = int(rng.integers(2304, 9217))   # at least 9 chunks
        out.append((B, int(rng.choice([4, 16])), lens, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,S,lens,dtype_f32", _many_chunk_cases(77, 6))
def test_many_chunk_merge(B, S, lens, dtype_f32):
    """Plans of more than 8 chunks per KV head (a few sequences, long ragged
    contexts: 9 to 36 chunks of 256 keys), where the merge folds 16 chunks
    per batch: sequences with fewer chunks than the batch, several batches,
    empty contexts, with the adaLN vectors and a residual; bf16 and fp32."""
    dtype = F32 if dtype_f32 else BF16
    c = attn_case(B, S, 32, 2, 128, lens, dtype=dtype, seed=sum(lens) + B + S, ada=True,
                  residual=True)
    _check(c, f"many chunks B={B} S={S}")
