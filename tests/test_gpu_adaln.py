"""GPU parity of the timestep embedding and adaLN-single against the oracle."""
import numpy as np
import pytest
import torch

import block_mask_diffusion_tt_amd as tt
import oracle
import synth

from .gpu_cases import DEV, np64, say

pytestmark = pytest.mark.gpu


def test_timestep_embed():
    t = torch.tensor([0.0, 1 / 16, 0.5, 10 / 16, 1.0, 3 / 7], dtype=torch.float32, device=DEV)
    emb = torch.empty((6, 256), dtype=torch.float32, device=DEV)
    say("timestep_embed", 6)
    tt.timestep_embed(6, t, emb)
    torch.cuda.synchronize()
    ref = oracle.timestep_embedding(np64(t))
    assert np.abs(np64(emb) - ref).max() < 1e-6


@pytest.mark.parametrize("B,width,n_layers", [(1, 4096, 6), (5, 256, 2), (130, 4096, 6)])
def test_adaln_single(B, width, n_layers):
    say("adaln_single", B, width, n_layers)
    emb = synth.normal((B, 256), 1.0, 1, torch.float32, DEV)          # random 256-d embedding
    w = synth.normal((256, 3 * width), 0.05, 2, torch.bfloat16, DEV)
    bias = synth.normal((3 * width,), 0.1, 3, torch.float32, DEV)
    table = synth.normal((n_layers, 3, width), 0.1, 4, torch.float32, DEV)
    ada = torch.empty((n_layers, 3, B, width), dtype=torch.float32, device=DEV)
    tt.adaln_single(B, width, n_layers, emb, w, bias, table, ada)
    torch.cuda.synchronize()
    ref = oracle.adaln_single(np64(emb), np64(w), np64(bias), np64(table))
    np.testing.assert_allclose(np64(ada), ref, rtol=1e-5, atol=2e-6)
    # without bias and table
    tt.adaln_single(B, width, n_layers, emb, w, None, None, ada)
    torch.cuda.synchronize()
    ref0 = oracle.adaln_single(np64(emb), np64(w), np.zeros(3 * width), np.zeros((n_layers, 3, width)))
    np.testing.assert_allclose(np64(ada), ref0, rtol=1e-5, atol=2e-6)


@pytest.mark.parametrize("B,width,n_layers", [(33, 260, 17), (2, 4, 1), (64, 4096, 6)])
def test_adaln_single_edges(B, width, n_layers):
    """Ragged tiles (33 sequences, 780 columns), a width that is not a
    multiple of 8, more layers than the kernel preloads table rows for, one
    layer, and an embedding that is 4-byte but not 16-byte aligned (a view one
    float into a larger buffer, which the interface allows)."""
    say("adaln_single edges", B, width, n_layers)
    buf = synth.normal((B * 256 + 1,), 1.0, 11, torch.float32, DEV)
    emb = buf[1:].view(B, 256)
    assert emb.data_ptr() % 16 == 4
    w = synth.normal((256, 3 * width), 0.05, 12, torch.bfloat16, DEV)
    bias = synth.normal((3 * width,), 0.1, 13, torch.float32, DEV)
    table = synth.normal((n_layers, 3, width), 0.1, 14, torch.float32, DEV)
    ada = torch.full((n_layers, 3, B, width), 7.0, dtype=torch.float32, device=DEV)
    tt.adaln_single(B, width, n_layers, emb, w, bias, table, ada)
    torch.cuda.synchronize()
    ref = oracle.adaln_single(np64(emb), np64(w), np64(bias), np64(table))
    np.testing.assert_allclose(np64(ada), ref, rtol=1e-5, atol=2e-6)


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(rng.integers(1, 201)), 4 * int(rng.integers(1, 257)),
                    int(rng.integers(1, 21)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,width,n_layers,has_bias,has_table", _shapes(2024, 6))
def test_adaln_single_random_shapes(B, width, n_layers, has_bias, has_table):
    """Seeded shapes across the kernel's tiling: batches that end mid-tile
    (32 sequences per tile), widths whose 3 * width columns end mid-tile (128
    per tile), layer counts on both sides of the 16 whose table rows are
    loaded up front, and a missing bias or table."""
    say("adaln_single random", B, width, n_layers, has_bias, has_table)
    seed = B * 7919 + width * 31 + n_layers
    emb = synth.normal((B, 256), 1.0, seed, torch.float32, DEV)
    w = synth.normal((256, 3 * width), 0.05, seed + 1, torch.bfloat16, DEV)
    bias = synth.normal((3 * width,), 0.1, seed + 2, torch.float32, DEV) if has_bias else None
    table = synth.normal((n_layers, 3, width), 0.1, seed + 3, torch.float32, DEV) if has_table else None
    ada = torch.full((n_layers, 3, B, width), 7.0, dtype=torch.float32, device=DEV)
    tt.adaln_single(B, width, n_layers, emb, w, bias, table, ada)
    torch.cuda.synchronize()
    ref = oracle.adaln_single(np64(emb), np64(w),
                              np64(bias) if has_bias else np.zeros(3 * width),
                              np64(table) if has_table else np.zeros((n_layers, 3, width)))
    np.testing.assert_allclose(np64(ada), ref, rtol=1e-5, atol=2e-6)
