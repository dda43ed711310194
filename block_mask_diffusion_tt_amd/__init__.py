"""MI355X-native block-denoising step of a two-tower block mask-diffusion
language model: hand-written gfx950 HIP kernels behind the C ABI of
include/tt.h (libtt.so), with a thin ctypes binding.  torch provides device
memory and streams only.  Importing this package requires the built library;
there is no CPU fallback."""
from ._binding import *  # noqa: F401,F403
from ._binding import (AttnShape, StepProvider, TTError, abi_version, adaln_single,  # noqa: F401
                       attn_shape, block_attn, block_attn_noalloc, block_attn_workspace_size, confidence_unmask,
                       ctx_advance, ctx_block_attn, sample_unmask, generate,
                       generate_workspace_size, GenProvider, mamba_shape, mamba_block_scan,
                       mamba_workspace_size,
                       MambaShape, ln_modulate, qkv_proj, out_proj,
                       adaln_sublayer_workspace_size, adaln_attn_sublayer,
                       denoise_block, denoise_block_resume, denoise_workspace_size, dtype_code,
                       last_error, lib,
                       timestep_embed, unmask_workspace_size, workspace_clear, EXPORTED,
                       LIB_PATH, TT_BF16, TT_F32)
