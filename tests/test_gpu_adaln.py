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
