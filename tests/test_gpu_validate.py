"""TT_VALIDATE: the device-side checks of the context arrays.  With the
variable set, valid calls give the same bits as without it, and each rule
(negative length or start, a context beyond its reserved region, two
overlapping regions) is reported as TT_ERR_INVALID_ARG before anything else of
the call runs.  Invalid arrays are only ever passed with the checks on, so no
compute kernel sees them."""
import pytest
import torch

import block_mask_diffusion_tt_amd as tt

from .gpu_cases import DEV, attn_case, run_attn, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("TT_VALIDATE", "1")


def _expect_invalid(fn, what, *args, **kw):
    with pytest.raises(tt.TTError) as ei:
        fn(*args, **kw)
    assert ei.value.status == tt.TT_ERR_INVALID_ARG
    msg = tt.last_error()
    say(what, msg)
    assert "TT_VALIDATE" in msg
    return msg


def test_valid_calls_unchanged(monkeypatch):
    c = attn_case(5, 16, 32, 2, 128, [300, 0, 4097, 64, 1000], seed=4100, ada=True,
                  active=[1, 1, 0, 1, 1])
    ref, ref_lse = run_attn(c)
    monkeypatch.setenv("TT_VALIDATE", "1")
    out, lse = run_attn(c)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_negative_length_and_start(validate):
    c = attn_case(4, 16, 8, 2, 64, [100, 50, 70, 20], seed=4200)
    c["ctx_len"][2] = -3
    shape = tt.attn_shape(4, 8, 2, 64, 16, torch.bfloat16)
    ws = torch.zeros(tt.block_attn_workspace_size(shape, 100), dtype=torch.uint8, device=DEV)
    out = torch.full((4, 16, 8, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    msg = _expect_invalid(tt.block_attn, "negative length", shape, c["q"], c["kb"], c["vb"],
                          c["kc"], c["vc"], c["ctx_start"], c["ctx_len"], 100, out, ws)
    assert "ctx_len[2] = -3" in msg
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)                       # nothing was launched
    # an inactive sequence is not checked
    active = torch.tensor([1, 1, 0, 1], dtype=torch.uint8, device=DEV)
    tt.block_attn(shape, c["q"], c["kb"], c["vb"], c["kc"], c["vc"], c["ctx_start"],
                  c["ctx_len"], 100, out, ws, active=active)
    torch.cuda.synchronize()
    c["ctx_len"][2] = 70
    # a start of -64 rows: the caches are views 64 rows into larger buffers,
    # so even those rows would be real memory
    kpad = torch.zeros((64 + c["kc"].shape[0], 2, 64), dtype=torch.bfloat16, device=DEV)
    vpad = torch.zeros_like(kpad)
    kpad[64:] = c["kc"]
    vpad[64:] = c["vc"]
    c["ctx_start"][1] = -64
    msg = _expect_invalid(tt.block_attn_noalloc, "negative start", shape, c["q"], c["kb"],
                          c["vb"], kpad[64:], vpad[64:], c["ctx_start"], c["ctx_len"], 100, out)
    assert "ctx_start[1] = -64" in msg


def test_regions_for_the_append(validate):
    c = attn_case(3, 16, 8, 2, 64, [40, 30, 20], seed=4300, gap=40)
    st = c["ctx_start"].cpu()
    shape = tt.attn_shape(3, 8, 2, 64, 16, torch.bfloat16)
    ws = torch.zeros(tt.block_attn_workspace_size(shape, 40), dtype=torch.uint8, device=DEV)
    out = torch.empty((3, 16, 8, 64), dtype=torch.bfloat16, device=DEV)
    lens = torch.tensor(c["lens"])
    # sequence 1's context does not fit its region
    end = (st + lens + 16).to(DEV)
    end[1] = st[1] + 10
    msg = _expect_invalid(tt.ctx_block_attn, "context beyond its region", shape, c["q"], c["kb"],
                          c["vb"], c["kc"], c["vc"], c["ctx_start"], c["ctx_len"], 40, out, ws,
                          ctx_end=end)
    assert "ctx_end[1]" in msg
    # sequence 0's region reaches into sequence 1's
    end = (st + lens + 16).to(DEV)
    end[0] = st[1] + 1
    msg = _expect_invalid(tt.ctx_block_attn, "overlapping regions", shape, c["q"], c["kb"],
                          c["vb"], c["kc"], c["vc"], c["ctx_start"], c["ctx_len"], 40, out, ws,
                          ctx_end=end)
    assert "sequences 0 and 1 overlap" in msg
    msg = _expect_invalid(tt.ctx_advance, "advance with overlapping regions", 3, 16,
                          c["ctx_start"], end, c["ctx_len"])
    assert "overlap" in msg
    # valid regions pass, and the call does its work
    end = (st + lens + 16).to(DEV)
    tt.ctx_block_attn(shape, c["q"], c["kb"], c["vb"], c["kc"], c["vc"], c["ctx_start"],
                      c["ctx_len"], 40, out, ws, ctx_end=end)
    tt.ctx_advance(3, 16, c["ctx_start"], end, c["ctx_len"])
    torch.cuda.synchronize()
    assert c["ctx_len"].cpu().tolist() == [56, 46, 36]


def test_loops_check_before_the_provider(validate):
    B, S, Hq, Hkv, d, V, NL = 2, 16, 8, 2, 64, 512, 2
    c = attn_case(B, S, Hq, Hkv, d, [100, 60], seed=4400, gap=S)
    c["ctx_len"][1] = -1
    shape = tt.attn_shape(B, Hq, Hkv, d, S, torch.bfloat16)
    calls = []

    class Provider:
        def layer_inputs(self, *a):
            calls.append("layer")

        def logits(self, *a):
            calls.append("logits")

        def ctx_inputs(self, *a):
            calls.append("ctx")

    tokens = torch.full((B, S), 3, dtype=torch.int32, device=DEV)
    masked = torch.ones((B, S), dtype=torch.uint8, device=DEV)
    ws = torch.zeros(tt.denoise_workspace_size(shape, NL, 100, V), dtype=torch.uint8, device=DEV)
    msg = _expect_invalid(tt.denoise_block, "denoise loop", shape, NL, S, 0.8, 1.0, 3, V,
                          [c["kc"]] * NL, [c["vc"]] * NL, c["ctx_start"], c["ctx_len"], 100,
                          Provider(), tokens, masked, ws)
    assert "ctx_len[1] = -1" in msg and not calls
    c["ctx_len"][1] = 60
    end = (c["ctx_start"].cpu() + torch.tensor([100, 60]) + S).to(DEV)
    end[0] = c["ctx_start"][0] + 50
    out = torch.empty((B, S), dtype=torch.int32, device=DEV)
    n_gen = torch.empty((B,), dtype=torch.int32, device=DEV)
    gws = torch.zeros(tt.generate_workspace_size(shape, NL, 1, 100, V), dtype=torch.uint8,
                      device=DEV)
    msg = _expect_invalid(tt.generate, "generation loop", shape, NL, 1, S, 0.8, 1.0, 3, -1, V,
                          [c["kc"]] * NL, [c["vc"]] * NL, c["ctx_start"], end, c["ctx_len"], 100,
                          Provider(), out, n_gen, gws)
    assert "ctx_end[0]" in msg and not calls
