"""ctypes binding of libtt (include/tt.h): argument marshalling only.

Every function here has the name of a C entry point without the ``tt_``
prefix.  Tensors are torch tensors resident on the GPU (torch is used for
device memory and streams only); they are passed as raw pointers.  The
stream defaults to torch's current stream, so torch events recorded on it
time the library's kernels.  A non-zero status raises ``TTError`` with the
library's message.  There is no fallback: if libtt.so is missing the import
of this module fails.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtt.so")

TT_OK, TT_ERR_INVALID_ARG, TT_ERR_UNSUPPORTED, TT_ERR_WORKSPACE, TT_ERR_HIP, TT_ERR_CALLBACK = range(6)
TT_BF16, TT_F32 = 0, 1
TIMESTEP_DIM = 256

_STATUS_NAMES = {0: "TT_OK", 1: "TT_ERR_INVALID_ARG", 2: "TT_ERR_UNSUPPORTED",
                 3: "TT_ERR_WORKSPACE", 4: "TT_ERR_HIP", 5: "TT_ERR_CALLBACK"}

# Every symbol include/tt.h declares.
EXPORTED = ["tt_last_error", "tt_abi_version", "tt_block_attn_workspace_size", "tt_block_attn",
            "tt_block_attn_noalloc", "tt_workspace_clear", "tt_timestep_embed", "tt_adaln_single",
            "tt_unmask_workspace_size", "tt_confidence_unmask", "tt_denoise_workspace_size",
            "tt_denoise_block", "tt_denoise_block_resume", "tt_ctx_block_attn", "tt_ctx_advance", "tt_sample_unmask",
            "tt_generate_workspace_size", "tt_generate", "tt_mamba_workspace_size",
            "tt_mamba_block_scan", "tt_ln_modulate", "tt_qkv_proj", "tt_out_proj",
            "tt_adaln_sublayer_workspace_size", "tt_adaln_attn_sublayer"]


class TTError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class MambaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_LAYER_INPUTS = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p)
_LOGITS = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p)


class StepProvider(ctypes.Structure):
    _fields_ = [("user", ctypes.c_void_p), ("layer_inputs", _LAYER_INPUTS), ("logits", _LOGITS)]


_G_LAYER_INPUTS = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)
_G_LOGITS = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)
_G_CTX_INPUTS = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)


class GenProvider(ctypes.Structure):
    _fields_ = [("user", ctypes.c_void_p), ("layer_inputs", _G_LAYER_INPUTS),
                ("logits", _G_LOGITS), ("ctx_inputs", _G_CTX_INPUTS)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_mask_diffusion_tt_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    shp = ctypes.POINTER(AttnShape)
    sigs = {
        "tt_last_error": (ctypes.c_char_p, []),
        "tt_abi_version": (ctypes.c_int, []),
        "tt_block_attn_workspace_size": (sz, [shp, i32]),
        "tt_block_attn": (ctypes.c_int, [shp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                         vp, vp, vp, vp, sz, vp]),
        "tt_block_attn_noalloc": (ctypes.c_int, [shp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                                 vp, vp, vp, vp, vp]),
        "tt_ctx_block_attn": (ctypes.c_int, [shp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                             vp, vp, vp, sz, vp]),
        "tt_ctx_advance": (ctypes.c_int, [i32, i32, vp, vp, vp, vp, vp, vp]),
        "tt_workspace_clear": (ctypes.c_int, [vp, sz, vp]),
        "tt_timestep_embed": (ctypes.c_int, [i32, vp, vp, vp]),
        "tt_adaln_single": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "tt_unmask_workspace_size": (sz, [i32, i32, i32]),
        "tt_confidence_unmask": (ctypes.c_int, [i32, i32, i32, vp, i32, i64, f32, f32, i32, i32,
                                                vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tt_sample_unmask": (ctypes.c_int, [i32, i32, i32, vp, i32, i64, f32, f32, ctypes.c_uint64,
                                            i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                            vp]),
        "tt_denoise_workspace_size": (sz, [shp, i32, i32, i32]),
        "tt_generate_workspace_size": (sz, [shp, i32, i32, i32, i32]),
        "tt_mamba_workspace_size": (sz, [ctypes.POINTER(MambaShape)]),
        "tt_mamba_block_scan": (ctypes.c_int, [ctypes.POINTER(MambaShape), vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tt_ln_modulate": (ctypes.c_int, [shp, i32, vp, vp, vp, vp, vp, vp]),
        "tt_qkv_proj": (ctypes.c_int, [shp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "tt_out_proj": (ctypes.c_int, [shp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "tt_adaln_sublayer_workspace_size": (sz, [shp, i32, i32]),
        "tt_adaln_attn_sublayer": (ctypes.c_int, [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  vp, i32, vp, vp, vp, sz, vp]),
        "tt_generate": (ctypes.c_int, [shp, i32, i32, i32, f32, f32, i32, ctypes.c_uint64, i32,
                                       i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                       ctypes.POINTER(GenProvider), vp, vp, vp,
                                       ctypes.POINTER(i32), vp, sz, vp]),
        "tt_denoise_block": (ctypes.c_int, [shp, i32, i32, f32, f32, i32, i32, vp, vp, vp, vp,
                                            i32, vp, vp, vp, ctypes.POINTER(StepProvider), vp,
                                            vp, vp, ctypes.POINTER(i32), vp, sz, vp]),
        "tt_denoise_block_resume": (ctypes.c_int, [shp, i32, i32, i32, f32, f32, i32,
                                                   ctypes.c_uint64, i32, i32, i32, vp, vp, vp,
                                                   vp, i32, vp, vp, vp,
                                                   ctypes.POINTER(StepProvider), vp, vp, vp,
                                                   ctypes.POINTER(i32), vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def last_error():
    return _lib.tt_last_error().decode()


def abi_version():
    return _lib.tt_abi_version()


def _check(status):
    if status != TT_OK:
        raise TTError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _on_stream(st):
    """A torch stream context for the library's hipStream_t `st` (0 / None:
    the null stream), so that a provider's copies are ordered with the
    library's launches on that stream."""
    if not st:
        return torch.cuda.stream(torch.cuda.default_stream())
    return torch.cuda.stream(torch.cuda.ExternalStream(st))


def dtype_code(dtype):
    if dtype == torch.bfloat16:
        return TT_BF16
    if dtype == torch.float32:
        return TT_F32
    raise ValueError(f"unsupported dtype {dtype}")


def attn_shape(batch, n_q_heads, n_kv_heads, head_dim, block_size, dtype):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return AttnShape(batch, n_q_heads, n_kv_heads, head_dim, block_size, code)


def block_attn_workspace_size(shape, max_ctx_len):
    n = _lib.tt_block_attn_workspace_size(ctypes.byref(shape), int(max_ctx_len))
    if n == 0:
        raise TTError(TT_ERR_INVALID_ARG, last_error())
    return n


def block_attn(shape, q_blk, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, max_ctx_len,
               out, workspace, active=None, ada_shift=None, ada_scale=None, ada_gate=None,
               residual=None, lse=None, stream=None):
    _check(_lib.tt_block_attn(ctypes.byref(shape), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk),
                              _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len),
                              int(max_ctx_len), _ptr(active), _ptr(ada_shift), _ptr(ada_scale),
                              _ptr(ada_gate), _ptr(residual), _ptr(out), _ptr(lse),
                              _ptr(workspace), _nbytes(workspace), _stream(stream)))


def block_attn_noalloc(shape, q_blk, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, max_ctx_len,
                       out, active=None, ada_shift=None, ada_scale=None, ada_gate=None,
                       residual=None, lse=None, stream=None):
    _check(_lib.tt_block_attn_noalloc(ctypes.byref(shape), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk),
                                      _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len),
                                      int(max_ctx_len), _ptr(active), _ptr(ada_shift),
                                      _ptr(ada_scale), _ptr(ada_gate), _ptr(residual), _ptr(out),
                                      _ptr(lse), _stream(stream)))


def ctx_block_attn(shape, q_blk, k_blk, v_blk, k_ctx, v_ctx, ctx_start, ctx_len, max_ctx_len,
                   out, workspace, ctx_end=None, active=None, residual=None, lse=None,
                   stream=None):
    _check(_lib.tt_ctx_block_attn(ctypes.byref(shape), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk),
                                  _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len),
                                  _ptr(ctx_end), int(max_ctx_len), _ptr(active), _ptr(residual),
                                  _ptr(out), _ptr(lse), _ptr(workspace), _nbytes(workspace),
                                  _stream(stream)))


def ctx_advance(batch, block_size, ctx_start, ctx_end, ctx_len, active=None, appended=None,
                stream=None):
    _check(_lib.tt_ctx_advance(int(batch), int(block_size), _ptr(ctx_start), _ptr(ctx_end),
                               _ptr(ctx_len), _ptr(active), _ptr(appended), _stream(stream)))


def workspace_clear(workspace, nbytes=None, stream=None):
    n = _nbytes(workspace) if nbytes is None else int(nbytes)
    _check(_lib.tt_workspace_clear(_ptr(workspace), n, _stream(stream)))


def timestep_embed(batch, t, emb, stream=None):
    _check(_lib.tt_timestep_embed(int(batch), _ptr(t), _ptr(emb), _stream(stream)))


def adaln_single(batch, width, n_layers, t_emb, w, bias, table, ada, stream=None):
    _check(_lib.tt_adaln_single(int(batch), int(width), int(n_layers), _ptr(t_emb), _ptr(w),
                                _ptr(bias), _ptr(table), _ptr(ada), _stream(stream)))


def unmask_workspace_size(batch, block_size, vocab):
    n = _lib.tt_unmask_workspace_size(int(batch), int(block_size), int(vocab))
    if n == 0:
        raise TTError(TT_ERR_INVALID_ARG, last_error())
    return n


def confidence_unmask(batch, block_size, vocab, logits, row_stride, gamma, temperature,
                      mask_token_id, step, tokens, masked, workspace, committed_now=None,
                      conf=None, pred=None, commit_step=None, n_masked=None, dtype=None,
                      stream=None):
    code = dtype_code(logits.dtype) if dtype is None else dtype
    _check(_lib.tt_confidence_unmask(int(batch), int(block_size), int(vocab), _ptr(logits), code,
                                     int(row_stride), float(gamma), float(temperature),
                                     int(mask_token_id), int(step), _ptr(tokens), _ptr(masked),
                                     _ptr(committed_now), _ptr(conf), _ptr(pred),
                                     _ptr(commit_step), _ptr(n_masked), _ptr(workspace),
                                     _nbytes(workspace), _stream(stream)))


def sample_unmask(batch, block_size, vocab, logits, row_stride, gamma, temperature, seed,
                  block_index, mask_token_id, step, tokens, masked, workspace, committed_now=None,
                  conf=None, pred=None, commit_step=None, n_masked=None, dtype=None, stream=None):
    code = dtype_code(logits.dtype) if dtype is None else dtype
    _check(_lib.tt_sample_unmask(int(batch), int(block_size), int(vocab), _ptr(logits), code,
                                 int(row_stride), float(gamma), float(temperature), int(seed),
                                 int(block_index), int(mask_token_id), int(step), _ptr(tokens),
                                 _ptr(masked), _ptr(committed_now), _ptr(conf), _ptr(pred),
                                 _ptr(commit_step), _ptr(n_masked), _ptr(workspace),
                                 _nbytes(workspace), _stream(stream)))


def denoise_workspace_size(shape, n_layers, max_ctx_len, vocab):
    n = _lib.tt_denoise_workspace_size(ctypes.byref(shape), int(n_layers), int(max_ctx_len),
                                       int(vocab))
    if n == 0:
        raise TTError(TT_ERR_INVALID_ARG, last_error())
    return n


def _nbytes(t):
    if t is None:
        return 0
    return t.numel() * t.element_size()


def denoise_block(shape, n_layers, max_steps, gamma, temperature, mask_token_id, vocab,
                  k_ctx_layers, v_ctx_layers, ctx_start, ctx_len, max_ctx_len, provider,
                  tokens, masked, workspace, commit_step=None, ada_w=None, ada_bias=None,
                  ada_table=None, stream=None):
    """Runs tt_denoise_block (see denoise_block_resume for the provider)."""
    return _denoise(None, shape, n_layers, max_steps, gamma, temperature, mask_token_id, vocab,
                    k_ctx_layers, v_ctx_layers, ctx_start, ctx_len, max_ctx_len, provider,
                    tokens, masked, workspace, commit_step, ada_w, ada_bias, ada_table, stream)


def denoise_block_resume(shape, n_layers, first_step, max_steps, gamma, temperature,
                         mask_token_id, vocab, k_ctx_layers, v_ctx_layers, ctx_start, ctx_len,
                         max_ctx_len, provider, tokens, masked, workspace, commit_step=None,
                         seed=None, block_index=0, ada_w=None, ada_bias=None, ada_table=None,
                         stream=None):
    """Runs tt_denoise_block_resume: steps first_step .. first_step+max_steps-1
    (seed None: argmax predictions; else temperature sampling with that seed
    and block_index).  Returns the number of steps this call ran."""
    resume = (int(first_step), 0 if seed is None else 1, 0 if seed is None else int(seed),
              int(block_index))
    return _denoise(resume, shape, n_layers, max_steps, gamma, temperature, mask_token_id, vocab,
                    k_ctx_layers, v_ctx_layers, ctx_start, ctx_len, max_ctx_len, provider,
                    tokens, masked, workspace, commit_step, ada_w, ada_bias, ada_table, stream)


def _denoise(resume, shape, n_layers, max_steps, gamma, temperature, mask_token_id, vocab,
             k_ctx_layers, v_ctx_layers, ctx_start, ctx_len, max_ctx_len, provider, tokens,
             masked, workspace, commit_step, ada_w, ada_bias, ada_table, stream):
    """The loop of tt_denoise_block (resume None) or of tt_denoise_block_resume
    (resume = (first_step, sample, seed, block_index)).  `provider` has two
    methods, called from inside the loop with tensor views of the library's
    workspace buffers:
        provider.layer_inputs(step, layer, prev_out, q_blk, k_blk, v_blk)
        provider.logits(step, last_out, logits)
    each filling its output tensors in place on the current stream, which is
    the library's stream while a callback runs (prev_out is None for layer
    0).  Returns the number of steps taken."""
    B, S, Hq, Hkv, d = shape.batch, shape.block_size, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    tdtype = torch.bfloat16 if shape.dtype == TT_BF16 else torch.float32
    esz = 2 if shape.dtype == TT_BF16 else 4
    ws_u8 = workspace.view(torch.uint8) if workspace.dtype != torch.uint8 else workspace
    base = workspace.data_ptr()

    def view(ptr, shape_):
        if not ptr:
            return None
        n = 1
        for x in shape_:
            n *= x
        off = ptr - base
        return ws_u8[off:off + n * esz].view(tdtype).view(*shape_)

    errors = []

    def _layer_inputs(user, step, layer, prev_out, q, kb, vb, st):
        try:
            with _on_stream(st):
                provider.layer_inputs(int(step), int(layer), view(prev_out, (B, S, Hq, d)),
                                      view(q, (B, S, Hq, d)), view(kb, (B, S, Hkv, d)),
                                      view(vb, (B, S, Hkv, d)))
            return 0
        except Exception as e:  # reported through TT_ERR_CALLBACK
            errors.append(e)
            return 1

    def _logits(user, step, last_out, lg, st):
        try:
            with _on_stream(st):
                provider.logits(int(step), view(last_out, (B, S, Hq, d)), view(lg, (B, S, vocab)))
            return 0
        except Exception as e:
            errors.append(e)
            return 1

    cb = StepProvider(None, _LAYER_INPUTS(_layer_inputs), _LOGITS(_logits))
    kptrs = (ctypes.c_void_p * n_layers)(*[_ptr(t) for t in k_ctx_layers])
    vptrs = (ctypes.c_void_p * n_layers)(*[_ptr(t) for t in v_ctx_layers])
    taken = ctypes.c_int32(0)
    rest = (int(mask_token_id), int(vocab), kptrs, vptrs, _ptr(ctx_start), _ptr(ctx_len),
            int(max_ctx_len), _ptr(ada_w), _ptr(ada_bias), _ptr(ada_table), ctypes.byref(cb),
            _ptr(tokens), _ptr(masked), _ptr(commit_step), ctypes.byref(taken), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    if resume is None:
        status = _lib.tt_denoise_block(ctypes.byref(shape), int(n_layers), int(max_steps),
                                       float(gamma), float(temperature), *rest)
    else:
        first, sample, seed, blk = resume
        status = _lib.tt_denoise_block_resume(ctypes.byref(shape), int(n_layers), first,
                                              int(max_steps), float(gamma), float(temperature),
                                              sample, seed, blk, *rest)
    if status != TT_OK:
        msg = last_error()
        if errors:
            msg += f" ({errors[0]!r})"
        raise TTError(status, msg)
    return taken.value


def generate_workspace_size(shape, n_layers, n_blocks, max_ctx_len, vocab):
    n = _lib.tt_generate_workspace_size(ctypes.byref(shape), int(n_layers), int(n_blocks),
                                        int(max_ctx_len), int(vocab))
    if n == 0:
        raise TTError(TT_ERR_INVALID_ARG, last_error())
    return n


def generate(shape, n_layers, n_blocks, steps_per_block, gamma, temperature, mask_token_id,
             eos_token_id, vocab, k_ctx_layers, v_ctx_layers, ctx_start, ctx_end, ctx_len,
             max_ctx_len, provider, out_tokens, n_generated, workspace, stop_reason=None,
             seed=None, ada_w=None, ada_bias=None, ada_table=None, stream=None):
    """Runs tt_generate (seed None: argmax predictions; else temperature
    sampling with that seed).  `provider` has three methods, called from
    inside the loop with tensor views of the library's workspace buffers:
        provider.layer_inputs(block, step, layer, prev_out, q_blk, k_blk, v_blk)
        provider.logits(block, step, last_out, logits)
        provider.ctx_inputs(block, layer, tokens, prev_out, q_blk, k_blk, v_blk)
    each filling its output tensors in place on the current stream, which is
    the library's stream while a callback runs (prev_out is None for layer
    0; tokens is the committed block [B, S] int32).
    Returns the number of blocks taken."""
    B, S, Hq, Hkv, d = shape.batch, shape.block_size, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    tdtype = torch.bfloat16 if shape.dtype == TT_BF16 else torch.float32
    ws_u8 = workspace.view(torch.uint8) if workspace.dtype != torch.uint8 else workspace
    base = workspace.data_ptr()

    def view(ptr, shape_, dt=tdtype):
        if not ptr:
            return None
        n = 1
        for x in shape_:
            n *= x
        off = ptr - base
        esz = torch.empty((), dtype=dt).element_size()
        return ws_u8[off:off + n * esz].view(dt).view(*shape_)

    errors = []

    def _wrap(fn):
        def inner(*a):
            try:
                with _on_stream(a[-1]):   # the library's stream is the last argument
                    fn(*a)
                return 0
            except Exception as e:  # reported through TT_ERR_CALLBACK
                errors.append(e)
                return 1
        return inner

    @_wrap
    def _layer_inputs(user, blk, step, layer, prev, q, kb, vb, st):
        provider.layer_inputs(int(blk), int(step), int(layer), view(prev, (B, S, Hq, d)),
                              view(q, (B, S, Hq, d)), view(kb, (B, S, Hkv, d)),
                              view(vb, (B, S, Hkv, d)))

    @_wrap
    def _logits(user, blk, step, last, lg, st):
        provider.logits(int(blk), int(step), view(last, (B, S, Hq, d)), view(lg, (B, S, vocab)))

    @_wrap
    def _ctx_inputs(user, blk, layer, toks, prev, q, kb, vb, st):
        provider.ctx_inputs(int(blk), int(layer), view(toks, (B, S), torch.int32),
                            view(prev, (B, S, Hq, d)), view(q, (B, S, Hq, d)),
                            view(kb, (B, S, Hkv, d)), view(vb, (B, S, Hkv, d)))

    cb = GenProvider(None, _G_LAYER_INPUTS(_layer_inputs), _G_LOGITS(_logits),
                     _G_CTX_INPUTS(_ctx_inputs))
    kptrs = (ctypes.c_void_p * n_layers)(*[_ptr(t) for t in k_ctx_layers])
    vptrs = (ctypes.c_void_p * n_layers)(*[_ptr(t) for t in v_ctx_layers])
    taken = ctypes.c_int32(0)
    status = _lib.tt_generate(ctypes.byref(shape), int(n_layers), int(n_blocks),
                              int(steps_per_block), float(gamma), float(temperature),
                              0 if seed is None else 1, 0 if seed is None else int(seed),
                              int(mask_token_id), int(eos_token_id), int(vocab), kptrs, vptrs,
                              _ptr(ctx_start), _ptr(ctx_end), _ptr(ctx_len), int(max_ctx_len),
                              _ptr(ada_w), _ptr(ada_bias), _ptr(ada_table), ctypes.byref(cb),
                              _ptr(out_tokens), _ptr(n_generated), _ptr(stop_reason),
                              ctypes.byref(taken), _ptr(workspace), _nbytes(workspace),
                              _stream(stream))
    if status != TT_OK:
        msg = last_error()
        if errors:
            msg += f" ({errors[0]!r})"
        raise TTError(status, msg)
    return taken.value


def mamba_shape(batch, n_heads, head_dim, d_state, n_groups, conv_width, block_size, dtype):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return MambaShape(batch, n_heads, head_dim, d_state, n_groups, conv_width, block_size, code)


def mamba_workspace_size(shape):
    n = _lib.tt_mamba_workspace_size(ctypes.byref(shape))
    if n == 0:
        raise TTError(TT_ERR_INVALID_ARG, last_error())
    return n


def mamba_block_scan(shape, xbc, dt_raw, conv_state, ssm_state, conv_w, A_log, y, workspace,
                     conv_b=None, dt_bias=None, D=None, active=None, conv_state_out=None,
                     ssm_state_out=None, stream=None):
    _check(_lib.tt_mamba_block_scan(ctypes.byref(shape), _ptr(xbc), _ptr(dt_raw), _ptr(conv_state),
                                    _ptr(ssm_state), _ptr(conv_w), _ptr(conv_b), _ptr(A_log),
                                    _ptr(dt_bias), _ptr(D), _ptr(active), _ptr(y),
                                    _ptr(conv_state_out), _ptr(ssm_state_out), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)))


# ---------------------------------------------------- weighted adaLN sublayer

def ln_modulate(shape, width, x, shift, scale, h, active=None, stream=None):
    _check(_lib.tt_ln_modulate(ctypes.byref(shape), int(width), _ptr(x), _ptr(shift), _ptr(scale),
                               _ptr(active), _ptr(h), _stream(stream)))


def qkv_proj(shape, width, h, w_qkv, q_blk, k_blk, v_blk, active=None, stream=None):
    _check(_lib.tt_qkv_proj(ctypes.byref(shape), int(width), _ptr(h), _ptr(w_qkv), _ptr(active),
                            _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _stream(stream)))


def out_proj(shape, width, o, w_o, gate, x, out, active=None, stream=None):
    _check(_lib.tt_out_proj(ctypes.byref(shape), int(width), _ptr(o), _ptr(w_o), _ptr(gate),
                            _ptr(x), _ptr(active), _ptr(out), _stream(stream)))


def adaln_sublayer_workspace_size(shape, width, max_ctx_len):
    n = _lib.tt_adaln_sublayer_workspace_size(ctypes.byref(shape), int(width), int(max_ctx_len))
    if n == 0:
        raise TTError(TT_ERR_INVALID_ARG, last_error())
    return n


def adaln_attn_sublayer(shape, width, x, shift, scale, gate, w_qkv, w_o, k_ctx, v_ctx, ctx_start,
                        ctx_len, max_ctx_len, out, workspace, active=None, stream=None):
    _check(_lib.tt_adaln_attn_sublayer(ctypes.byref(shape), int(width), _ptr(x), _ptr(shift),
                                       _ptr(scale), _ptr(gate), _ptr(w_qkv), _ptr(w_o), _ptr(k_ctx),
                                       _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len),
                                       int(max_ctx_len), _ptr(active), _ptr(out), _ptr(workspace),
                                       _nbytes(workspace), _stream(stream)))
