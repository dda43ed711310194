"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and rejects invalid calls with the documented status before any
HIP call (these run without a GPU: validation returns before a launch)."""
import ctypes
import os
import re

import pytest

import block_mask_diffusion_tt_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a 256-byte-aligned non-NULL address; never dereferenced


def _header_functions():
    with open(os.path.join(ROOT, "include", "tt.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _header_functions()
    assert "tt_block_attn" in names and "tt_denoise_block" in names
    lib = ctypes.CDLL(tt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(tt.EXPORTED) == names


def test_abi_version():
    assert tt.abi_version() == 4


def _status(fn, *args):
    return fn(*args)


def _attn(shape, ws_bytes=1 << 30, **over):
    args = dict(q=FAKE, kb=FAKE, vb=FAKE, kc=FAKE, vc=FAKE, cs=FAKE, cl=FAKE, maxl=128,
                active=None, shift=None, scale=None, gate=None, res=None, out=FAKE, lse=None,
                ws=FAKE, stream=None)
    args.update(over)
    return tt.lib().tt_block_attn(ctypes.byref(shape), args["q"], args["kb"], args["vb"],
                                  args["kc"], args["vc"], args["cs"], args["cl"], args["maxl"],
                                  args["active"], args["shift"], args["scale"], args["gate"],
                                  args["res"], args["out"], args["lse"], args["ws"], ws_bytes,
                                  args["stream"])


@pytest.mark.parametrize("shape,status", [
    ((1, 32, 3, 128, 16, 0), tt.TT_ERR_INVALID_ARG),    # Hq % Hkv
    ((1, 32, 2, 96, 16, 0), tt.TT_ERR_UNSUPPORTED),     # head_dim 96
    ((1, 32, 2, 0, 16, 0), tt.TT_ERR_INVALID_ARG),      # head_dim 0
    ((1, 32, 2, 128, 0, 0), tt.TT_ERR_INVALID_ARG),     # S = 0
    ((1, 32, 2, 128, 65, 0), tt.TT_ERR_INVALID_ARG),    # S > 64
    ((1, 32, 2, 128, 16, 7), tt.TT_ERR_INVALID_ARG),    # dtype
    ((-1, 32, 2, 128, 16, 0), tt.TT_ERR_INVALID_ARG),   # batch < 0
    ((1, 0, 2, 128, 16, 0), tt.TT_ERR_INVALID_ARG),     # no heads
])
def test_block_attn_rejects_bad_shapes(shape, status):
    s = tt.AttnShape(*shape)
    assert _attn(s) == status
    assert tt.last_error() != ""


def test_block_attn_noalloc_rejects_bad_calls_before_any_launch():
    lib = tt.lib()

    def call(s, q=FAKE, maxl=128):
        return lib.tt_block_attn_noalloc(ctypes.byref(s), q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         maxl, None, None, None, None, None, FAKE, None, None)
    assert call(tt.AttnShape(1, 32, 3, 128, 16, 0)) == tt.TT_ERR_INVALID_ARG
    assert call(tt.AttnShape(2, 32, 2, 128, 16, 0), q=None) == tt.TT_ERR_INVALID_ARG
    assert call(tt.AttnShape(2, 32, 2, 128, 16, 0), maxl=-1) == tt.TT_ERR_INVALID_ARG
    # a launch whose partials exceed the 64 MiB scratch
    big = tt.AttnShape(2048, 64, 8, 128, 64, 0)
    assert tt.block_attn_workspace_size(big, 1 << 16) > (64 << 20)
    assert call(big, maxl=1 << 16) == tt.TT_ERR_WORKSPACE
    assert "scratch" in tt.last_error()
    # an empty batch is a no-op
    assert call(tt.AttnShape(0, 32, 2, 128, 16, 0)) == tt.TT_OK


def test_block_attn_rejects_bad_pointers_and_workspace():
    s = tt.AttnShape(2, 32, 2, 128, 16, 0)
    assert _attn(s, q=None) == tt.TT_ERR_INVALID_ARG
    assert _attn(s, cl=None) == tt.TT_ERR_INVALID_ARG
    assert _attn(s, q=FAKE + 2) == tt.TT_ERR_INVALID_ARG            # misaligned
    assert _attn(s, gate=FAKE + 4) == tt.TT_ERR_INVALID_ARG          # gate needs 16 B
    assert _attn(s, maxl=-1) == tt.TT_ERR_INVALID_ARG
    need = tt.block_attn_workspace_size(s, 128)
    assert _attn(s, ws_bytes=need - 1) == tt.TT_ERR_WORKSPACE
    assert _attn(s, ws=None) == tt.TT_ERR_WORKSPACE
    assert "workspace" in tt.last_error()


def test_block_attn_empty_batch_is_ok_without_gpu():
    s = tt.AttnShape(0, 32, 2, 128, 16, 0)
    assert _attn(s, ws_bytes=0, ws=None) == tt.TT_OK


def test_workspace_sizes_monotone():
    a = tt.block_attn_workspace_size(tt.attn_shape(8, 32, 2, 128, 16, 0), 1024)
    b = tt.block_attn_workspace_size(tt.attn_shape(8, 32, 2, 128, 16, 0), 32768)
    assert 0 < a <= b
    assert tt.unmask_workspace_size(64, 16, 131072) >= 64 * 16 * 16
    with pytest.raises(tt.TTError):
        tt.unmask_workspace_size(1, 0, 10)


def _unmask(B=1, S=16, V=1024, logits=FAKE, dtype=0, stride=None, gamma=0.8, tau=1.0,
            tokens=FAKE, masked=FAKE, ws=FAKE, ws_bytes=1 << 20):
    return tt.lib().tt_confidence_unmask(B, S, V, logits, dtype, V if stride is None else stride,
                                         gamma, tau, 3, 0, tokens, masked, None, None, None, None,
                                         None, ws, ws_bytes, None)


def test_unmask_rejects_bad_arguments():
    assert _unmask(S=0) == tt.TT_ERR_INVALID_ARG
    assert _unmask(S=65) == tt.TT_ERR_INVALID_ARG
    assert _unmask(V=0) == tt.TT_ERR_INVALID_ARG
    assert _unmask(stride=100) == tt.TT_ERR_INVALID_ARG
    assert _unmask(tau=0.0) == tt.TT_ERR_INVALID_ARG
    assert _unmask(tau=-1.0) == tt.TT_ERR_INVALID_ARG
    assert _unmask(tau=float("inf")) == tt.TT_ERR_INVALID_ARG
    assert _unmask(gamma=float("nan")) == tt.TT_ERR_INVALID_ARG
    assert _unmask(dtype=5) == tt.TT_ERR_INVALID_ARG
    assert _unmask(logits=None) == tt.TT_ERR_INVALID_ARG
    assert _unmask(tokens=None) == tt.TT_ERR_INVALID_ARG
    assert _unmask(ws_bytes=1) == tt.TT_ERR_WORKSPACE
    assert _unmask(B=0, ws=None, ws_bytes=0) == tt.TT_OK


def test_adaln_and_embed_reject_bad_arguments():
    L = tt.lib()
    assert L.tt_timestep_embed(-1, FAKE, FAKE, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_timestep_embed(2, None, FAKE, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_adaln_single(2, 6, 1, FAKE, FAKE, None, None, FAKE, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_adaln_single(2, 8, 0, FAKE, FAKE, None, None, FAKE, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_adaln_single(2, 8, 1, None, FAKE, None, None, FAKE, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_workspace_clear(None, 16, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_workspace_clear(None, 0, None) == tt.TT_OK


def test_denoise_rejects_bad_arguments():
    s = tt.AttnShape(2, 4, 1, 64, 16, 1)
    L = tt.lib()
    ptrs = (ctypes.c_void_p * 1)(FAKE)
    prov = tt.StepProvider()

    def call(shape=s, n_layers=1, max_steps=16, provider=None, k=ptrs, ws_bytes=1 << 30):
        taken = ctypes.c_int32(-5)
        st = L.tt_denoise_block(ctypes.byref(shape), n_layers, max_steps, 0.8, 1.0, 3, 64,
                                k, ptrs, FAKE, FAKE, 8, None, None, None,
                                provider, FAKE, FAKE, None, ctypes.byref(taken), FAKE,
                                ws_bytes, None)
        assert taken.value == 0
        return st
    assert call(max_steps=17) == tt.TT_ERR_INVALID_ARG
    assert call(max_steps=-1) == tt.TT_ERR_INVALID_ARG
    assert call(n_layers=0) == tt.TT_ERR_INVALID_ARG
    assert call(provider=None) == tt.TT_ERR_INVALID_ARG
    assert call(provider=ctypes.byref(prov)) == tt.TT_ERR_INVALID_ARG    # NULL callbacks
    assert call(k=(ctypes.c_void_p * 1)(None)) == tt.TT_ERR_INVALID_ARG
    assert tt.denoise_workspace_size(s, 1, 8, 64) > 0


def test_denoise_resume_rejects_bad_arguments():
    s = tt.AttnShape(2, 4, 1, 64, 16, 1)
    L = tt.lib()
    ptrs = (ctypes.c_void_p * 1)(FAKE)

    def call(first=0, max_steps=16, sample=0, block=0):
        taken = ctypes.c_int32(-5)
        st = L.tt_denoise_block_resume(ctypes.byref(s), 1, first, max_steps, 0.8, 1.0, sample, 9,
                                       block, 3, 64, ptrs, ptrs, FAKE, FAKE, 8, None, None, None,
                                       None, FAKE, FAKE, None, ctypes.byref(taken), FAKE, 1 << 30,
                                       None)
        assert taken.value == 0
        return st
    assert call(first=-1) == tt.TT_ERR_INVALID_ARG
    assert call(first=17, max_steps=0) == tt.TT_ERR_INVALID_ARG
    assert call(first=4, max_steps=13) == tt.TT_ERR_INVALID_ARG     # past the block's S steps
    assert call(first=4, max_steps=12, sample=1, block=-1) == tt.TT_ERR_INVALID_ARG
    assert "first_step" in tt.last_error() or "block_index" in tt.last_error()
    # in range: it gets as far as the NULL provider
    assert call(first=4, max_steps=12) == tt.TT_ERR_INVALID_ARG
    assert "provider" in tt.last_error()


def test_binding_raises_with_message():
    with pytest.raises(tt.TTError) as ei:
        tt.block_attn_workspace_size(tt.AttnShape(1, 3, 2, 64, 4, 0), 8)
    assert "multiple" in str(ei.value)


def _ctx_attn(shape, ws_bytes=1 << 30, **over):
    args = dict(q=FAKE, kb=FAKE, vb=FAKE, kc=FAKE, vc=FAKE, cs=FAKE, cl=FAKE, ce=FAKE, maxl=128,
                active=None, res=None, out=FAKE, lse=None, ws=FAKE, stream=None)
    args.update(over)
    return tt.lib().tt_ctx_block_attn(ctypes.byref(shape), args["q"], args["kb"], args["vb"],
                                      args["kc"], args["vc"], args["cs"], args["cl"], args["ce"],
                                      args["maxl"], args["active"], args["res"], args["out"],
                                      args["lse"], args["ws"], ws_bytes, args["stream"])


def test_ctx_block_attn_rejects_bad_arguments():
    s = tt.AttnShape(2, 32, 2, 128, 16, 0)
    assert _ctx_attn(tt.AttnShape(1, 32, 3, 128, 16, 0)) == tt.TT_ERR_INVALID_ARG
    assert _ctx_attn(tt.AttnShape(1, 32, 2, 96, 16, 0)) == tt.TT_ERR_UNSUPPORTED
    assert _ctx_attn(s, kc=None) == tt.TT_ERR_INVALID_ARG
    assert _ctx_attn(s, ce=FAKE + 4) == tt.TT_ERR_INVALID_ARG         # ctx_end needs 8 B
    assert _ctx_attn(s, vc=FAKE + 8) == tt.TT_ERR_INVALID_ARG         # cache needs 16 B
    assert _ctx_attn(s, maxl=-3) == tt.TT_ERR_INVALID_ARG
    need = tt.block_attn_workspace_size(s, 128)
    assert _ctx_attn(s, ws_bytes=need - 1) == tt.TT_ERR_WORKSPACE
    assert "tt_ctx_block_attn" in tt.last_error()
    assert _ctx_attn(tt.AttnShape(0, 32, 2, 128, 16, 0), ws=None, ws_bytes=0) == tt.TT_OK


def test_ctx_advance_rejects_bad_arguments():
    L = tt.lib()
    assert L.tt_ctx_advance(-1, 16, FAKE, FAKE, FAKE, None, None, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_ctx_advance(2, 0, FAKE, FAKE, FAKE, None, None, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_ctx_advance(2, 65, FAKE, FAKE, FAKE, None, None, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_ctx_advance(2, 16, FAKE, None, FAKE, None, None, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_ctx_advance(2, 16, FAKE, FAKE, FAKE + 2, None, None, None) == tt.TT_ERR_INVALID_ARG
    assert L.tt_ctx_advance(0, 16, FAKE, FAKE, FAKE, None, None, None) == tt.TT_OK


def test_sample_unmask_rejects_bad_arguments():
    L = tt.lib()

    def call(B=1, S=16, V=1024, logits=FAKE, tau=0.1, gamma=0.8, block=0, step=0, ws_bytes=1 << 20):
        return L.tt_sample_unmask(B, S, V, logits, 0, V, gamma, tau, 7, block, 3, step, FAKE, FAKE,
                                  None, None, None, None, None, FAKE, ws_bytes, None)
    assert call(S=0) == tt.TT_ERR_INVALID_ARG
    assert call(tau=0.0) == tt.TT_ERR_INVALID_ARG
    assert call(gamma=float("nan")) == tt.TT_ERR_INVALID_ARG
    assert call(block=-1) == tt.TT_ERR_INVALID_ARG
    assert call(step=-2) == tt.TT_ERR_INVALID_ARG
    assert call(logits=None) == tt.TT_ERR_INVALID_ARG
    assert call(ws_bytes=1) == tt.TT_ERR_WORKSPACE
    assert "tt_sample_unmask" in tt.last_error()
    assert call(B=0) == tt.TT_OK


def test_generate_rejects_bad_arguments():
    s = tt.AttnShape(2, 4, 1, 64, 16, 0)
    L = tt.lib()
    ptrs = (ctypes.c_void_p * 1)(FAKE)
    prov = tt.GenProvider()

    def call(shape=s, n_layers=1, n_blocks=2, steps=16, provider=None, k=ptrs, ce=FAKE,
             out=FAKE, ws_bytes=1 << 30):
        taken = ctypes.c_int32(-5)
        st = L.tt_generate(ctypes.byref(shape), n_layers, n_blocks, steps, 0.8, 0.1, 1, 5, 3, 2,
                           64, k, ptrs, FAKE, ce, FAKE, 8, None, None, None, provider, out,
                           FAKE, None, ctypes.byref(taken), FAKE, ws_bytes, None)
        assert taken.value == 0
        return st
    assert call(steps=0) == tt.TT_ERR_INVALID_ARG
    assert call(steps=17) == tt.TT_ERR_INVALID_ARG
    assert call(n_blocks=-1) == tt.TT_ERR_INVALID_ARG
    assert call(n_layers=0) == tt.TT_ERR_INVALID_ARG
    assert call(provider=None) == tt.TT_ERR_INVALID_ARG
    assert call(provider=ctypes.byref(prov)) == tt.TT_ERR_INVALID_ARG    # NULL callbacks
    assert call(ce=None) == tt.TT_ERR_INVALID_ARG
    assert call(out=None) == tt.TT_ERR_INVALID_ARG
    assert call(k=(ctypes.c_void_p * 1)(None)) == tt.TT_ERR_INVALID_ARG
    assert "tt_generate" in tt.last_error()
    assert tt.generate_workspace_size(s, 1, 2, 8, 64) > tt.denoise_workspace_size(s, 1, 8, 64)


def test_mamba_rejects_bad_arguments():
    L = tt.lib()

    def call(shape=(2, 8, 64, 128, 2, 4, 16, 0), xbc=FAKE, ss=FAKE, cso=None, cs=FAKE,
             ws_bytes=1 << 30):
        s = tt.MambaShape(*shape)
        return L.tt_mamba_block_scan(ctypes.byref(s), xbc, FAKE, cs, ss, FAKE, None, FAKE, None,
                                     None, None, FAKE, cso, None, FAKE, ws_bytes, None)
    assert call(shape=(2, 8, 64, 128, 3, 4, 16, 0)) == tt.TT_ERR_INVALID_ARG     # G !| H
    assert call(shape=(2, 8, 48, 128, 2, 4, 16, 0)) == tt.TT_ERR_UNSUPPORTED     # P = 48
    assert call(shape=(2, 8, 64, 96, 2, 4, 16, 0)) == tt.TT_ERR_UNSUPPORTED      # N = 96
    assert call(shape=(2, 8, 64, 128, 2, 1, 16, 0)) == tt.TT_ERR_INVALID_ARG     # W = 1
    assert call(shape=(2, 8, 64, 128, 2, 6, 16, 0)) == tt.TT_ERR_UNSUPPORTED     # W = 6
    assert call(shape=(2, 8, 64, 128, 2, 4, 65, 0)) == tt.TT_ERR_INVALID_ARG     # S = 65
    assert call(shape=(2, 8, 64, 128, 2, 4, 16, 9)) == tt.TT_ERR_INVALID_ARG     # dtype
    assert call(xbc=None) == tt.TT_ERR_INVALID_ARG
    assert call(ss=FAKE + 8) == tt.TT_ERR_INVALID_ARG                            # 16-byte state
    assert call(cso=FAKE) == tt.TT_ERR_INVALID_ARG                               # overlaps conv_state
    assert "tt_mamba_block_scan" in tt.last_error()
    assert call(ws_bytes=16) == tt.TT_ERR_WORKSPACE
    assert call(shape=(0, 8, 64, 128, 2, 4, 16, 0)) == tt.TT_OK
    assert tt.mamba_workspace_size(tt.MambaShape(2, 8, 64, 128, 2, 4, 16, 0)) >= 2 * 2 * 16 * 272 * 4


def test_sublayer_rejects_bad_arguments():
    L = tt.lib()
    F2 = FAKE * 2                      # a second, disjoint fake buffer

    def shp(B=2, Hq=4, Hkv=2, d=64, S=16, dtype=0):
        return tt.AttnShape(B, Hq, Hkv, d, S, dtype)

    def ln(s=None, width=256, x=FAKE, h=F2):
        s = s or shp()
        return L.tt_ln_modulate(ctypes.byref(s), width, x, FAKE, FAKE, None, h, None)
    assert ln(s=shp(dtype=1)) == tt.TT_ERR_UNSUPPORTED                # fp32 storage
    assert ln(width=200) == tt.TT_ERR_UNSUPPORTED                     # not a multiple of 64
    assert ln(width=8256) == tt.TT_ERR_UNSUPPORTED                    # wider than 8192
    assert ln(x=None) == tt.TT_ERR_INVALID_ARG
    assert ln(h=F2 + 8) == tt.TT_ERR_INVALID_ARG                      # misaligned
    assert ln(h=FAKE + 256) == tt.TT_ERR_INVALID_ARG                  # partial overlap of x
    assert "tt_ln_modulate" in tt.last_error()
    assert ln(s=shp(B=0)) == tt.TT_OK

    def qkv(h=FAKE, q=F2, k=F2 * 2, v=F2 * 3):
        return L.tt_qkv_proj(ctypes.byref(shp()), 256, h, FAKE, None, q, k, v, None)
    assert qkv(h=None) == tt.TT_ERR_INVALID_ARG
    assert qkv(q=FAKE) == tt.TT_ERR_INVALID_ARG                       # q overlaps h

    def outp(o=FAKE, x=F2, out=F2 * 2):
        return L.tt_out_proj(ctypes.byref(shp()), 256, o, FAKE, FAKE, x, None, out, None)
    assert outp(out=FAKE) == tt.TT_ERR_INVALID_ARG                    # out overlaps o
    assert outp(out=F2 + 512) == tt.TT_ERR_INVALID_ARG                # partial overlap of x
    assert outp(o=FAKE + 4) == tt.TT_ERR_INVALID_ARG

    def sub(ws_bytes=1 << 30, maxl=64, out=F2):
        return L.tt_adaln_attn_sublayer(ctypes.byref(shp()), 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, maxl, None, out, FAKE, ws_bytes, None)
    assert sub(ws_bytes=256) == tt.TT_ERR_WORKSPACE
    assert sub(maxl=-1) == tt.TT_ERR_INVALID_ARG
    assert sub(out=F2 + 2) == tt.TT_ERR_INVALID_ARG
    n = L.tt_adaln_sublayer_workspace_size(ctypes.byref(shp()), 256, 64)
    assert n >= 2 * 16 * (256 + 2 * 256 + 2 * 128) * 2
    assert L.tt_adaln_sublayer_workspace_size(ctypes.byref(shp(dtype=1)), 256, 64) == 0
