"""tt_block_attn_noalloc (the attention entry point that allocates nothing
and keeps its partial results in the library's per-GPU scratch) against
tt_block_attn with a caller workspace, through the C ABI: identical bits, on
consecutive calls whose second input is smaller than the first (the scratch
keeps the previous call's contents)."""
import ctypes

import pytest
import torch

import block_mask_diffusion_tt_amd as tt

from .gpu_cases import attn_case, run_attn, say

pytestmark = pytest.mark.gpu


def _noalloc(c, stream=None):
    shape = tt.attn_shape(c["B"], c["Hq"], c["Hkv"], c["d"], c["S"], c["dtype"])
    out = torch.full((c["B"], c["S"], c["Hq"], c["d"]), 7.0, dtype=c["dtype"], device="cuda")
    lse = torch.full((c["B"], c["S"], c["Hq"]), 7.0, dtype=torch.float32, device="cuda")
    tt.block_attn_noalloc(shape, c["q"], c["kb"], c["vb"], c["kc"], c["vc"], c["ctx_start"],
                          c["ctx_len"], c["max_len"], out, active=c["active"],
                          ada_shift=c["shift"], ada_scale=c["scale"], ada_gate=c["gate"],
                          residual=c["residual"], lse=lse, stream=stream)
    torch.cuda.synchronize()
    return out, lse


def _same(c, what, stream=None):
    say(what, {k: c[k] for k in ("B", "S", "Hq", "Hkv", "d", "dtype")}, "lens", c["lens"][:8])
    out, lse = _noalloc(c, stream)
    ref_out, ref_lse = run_attn(c)
    assert torch.equal(out, ref_out), what
    assert torch.equal(lse, ref_lse), what


def test_noalloc_matches_workspace_call_twice():
    # the denoiser layer of 64 sequences x 8192 context tokens (bf16, adaLN,
    # residual), then a smaller fp32 call with a ragged and an empty context,
    # then a small bf16 call again: each is bit-identical to tt_block_attn
    big = attn_case(64, 16, 32, 2, 128, [8192] * 64, seed=900, ada=True, residual=True)
    _same(big, "noalloc headline layer")
    del big
    small = attn_case(3, 4, 8, 2, 64, [300, 0, 77], dtype=torch.float32, seed=910, ada=True)
    _same(small, "noalloc small fp32")
    side = torch.cuda.Stream()
    tiny = attn_case(2, 16, 32, 2, 128, [129, 5000], seed=920, ada=True, residual=True,
                     active=[1, 0])
    with torch.cuda.stream(side):
        _same(tiny, "noalloc small bf16 on a side stream", stream=side.cuda_stream)


def test_noalloc_rejects_launches_beyond_the_scratch():
    # 2048 sequences x 8 KV heads: the partials need more than the scratch
    s = tt.AttnShape(2048, 64, 8, 128, 64, 0)
    need = tt.block_attn_workspace_size(s, 1 << 16)
    assert need > (64 << 20)
    fake = 1 << 20
    st = tt.lib().tt_block_attn_noalloc(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake,
                                         1 << 16, None, None, None, None, None, fake, None, None)
    assert st == tt.TT_ERR_WORKSPACE
    assert "scratch" in tt.last_error()
