"""Oracle: a plain, slow, fp64 CPU definition of the block-denoising step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code,
constant table or helper with the HIP library under
``block_mask_diffusion_tt_amd/`` and never imports it; the product path never
imports this package.

Every function states the passage of the pages it follows.  Citation tags:

  [keyframe]  "Diffusion Nemotron: Nvidia's "Two Brain" Diffusion Model"
              (keyframe.defihacklabs.io video summary)
  [news]      "NVIDIA发布Nemotron两塔模型，实现2.42倍文本生成吞吐并保持98.7%质量"
              (889990.xyz)
  [telegram]  "NVIDIA, возможно, решила главный компромисс современных LLM"
              (tgviewer.app post)
  [dothoosh]  "فرآیند انتشار در برابر رمزگشایی متوالی در مدل جدید انویدیا"
              (dothoosh.com)
  [modelcard] "Nemotron-Labs-TwoTower-30B-A3B-Base-BF16" model-card digest
              (aitrends.kr)

What is pinned, and how (tests/test_oracle_*.py):
  attention      -- empty context reduces to torch's fp64 scaled-dot-product
                    attention; equals a dense block-causal masked attention over
                    the concatenated sequence; probability rows sum to one;
                    closed forms (single key, equal keys, planted key, zero
                    query); GQA == MHA with repeated heads; permutation
                    invariances; scalar-loop brute force on tiny shapes.
  unmasking      -- closed forms for p on hand-built logits (V=2, one planted
                    logit, temperature), the gamma threshold (inclusive), the
                    one-commit rule with lowest-position ties, lowest-id argmax
                    ties, monotonicity in gamma, loop invariants, scalar-loop
                    brute force.
  context tower  -- empty context reduces to torch's fp64 causal
                    scaled-dot-product attention; equals the dense block-causal
                    form with one block per new token; row s equals a one-token
                    decode step over [context ; block tokens < s]; the last row
                    equals the denoiser's bidirectional last row; rows ignore
                    later block keys; scalar-loop brute force; cache append and
                    length rule on hand-built regions (room, no room, inactive).
  sampling       -- Philox4x32-10 known-answer vectors; the uniform map's
                    range and fp32 exactness; Gumbel mean and variance; token
                    frequencies matching softmax(l / tau); closed forms of the
                    reported confidence; commit rule under sampling.
  generation     -- EOS stop and cache-room stop on hand-built logits; caches
                    holding the provider's K/V of every generated block in
                    order; the next block's attention equal to attention over
                    the explicit concatenation; every generated slot final.
  Mamba-2 seed   -- the recurrence equals the state-space duality's quadratic
                    form; context-then-seeded-block equals one scan of the
                    concatenation from zero states; the convolution against
                    numpy.convolve; closed forms (instant decay, zero step);
                    causality inside the block; brute force.
  weighted       -- LayerNorm against torch's fp64 layer_norm, its D = 2
  sublayer          closed form, zero mean / unit variance and affine
                    invariance; modulation special cases; selection weights
                    reducing the sublayer to the pinned block attention (q|k|v
                    column order, head reshape, O projection, gate); scalar-
                    loop brute force; block-slot permutation; gate = 0 and
                    W_o = 0 leave x.  The placement (the published
                    adaLN-single one) is a reading of the pages.
  adaLN-single   -- SiLU(0)=0, sinusoid special values, scalar-loop brute
                    force of the affine map.  The PLACEMENT of scale/shift/gate
                    and the timestep definition are readings the pages do not
                    fix: parity unpinned for those two choices.
"""

from .attention import (  # noqa: F401
    timestep_embedding,
    adaln_single,
    modulate_q,
    block_attn,
    dense_block_causal_attn,
)
from .context import (  # noqa: F401
    ctx_block_attn,
    kv_append,
    ctx_advance,
)
from .unmask import (  # noqa: F401
    row_confidence,
    confidence_unmask,
    denoise_block,
)
from .sampling import (  # noqa: F401
    philox4x32_10,
    uniform_words,
    gumbel_noise,
    row_sample,
)
from .generate import generate  # noqa: F401
from .sublayer import (  # noqa: F401
    layer_norm,
    ln_modulate,
    linear,
    split_qkv,
    gate_residual,
    adaln_attn_sublayer,
)
from .mamba import (  # noqa: F401
    causal_conv,
    mamba_block_scan,
    mamba_dual_form,
)
