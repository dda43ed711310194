"""Seeded synthetic inputs shared by the tests, the benchmark and smoke().

This module only draws random numbers with fixed seeds and shapes; it holds
none of the method's arithmetic.  Every tensor is produced with torch's
counter-based Philox generator (CUDA/HIP device) or its CPU generator, so a
(seed, shape, device) triple always yields the same bytes on that device.  The
oracle is always fed D2H copies of exactly the bytes the GPU consumed, so the
two devices never need to agree on the stream of random numbers.
"""

import torch


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std=1.0, seed=0, dtype=torch.bfloat16, device="cpu"):
    """N(0, std^2) samples (std is the standard deviation), rounded to dtype."""
    x = torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(float(std))
    return x.to(dtype)


def uniform_int(n, lo, hi, seed=0):
    """n integers uniform in [lo, hi] (inclusive), on the CPU, int64."""
    return torch.randint(int(lo), int(hi) + 1, (int(n),), generator=_gen(seed, "cpu"),
                         dtype=torch.int64)


def ragged_context(lengths):
    """Token offsets of sequences laid out back to back in one cache:
    returns (ctx_start int64 [B], ctx_len int32 [B], total tokens)."""
    lens = torch.as_tensor(lengths, dtype=torch.int64)
    start = torch.zeros_like(lens)
    if lens.numel() > 1:
        start[1:] = torch.cumsum(lens, 0)[:-1]
    return start, lens.to(torch.int32), int(lens.sum())


def masked_subset(batch, block, n_masked, seed=0):
    """uint8 [batch, block] bitmap with exactly n_masked ones per row, the
    positions drawn uniformly without replacement."""
    g = _gen(seed, "cpu")
    out = torch.zeros((batch, block), dtype=torch.uint8)
    for b in range(batch):
        idx = torch.randperm(block, generator=g)[:n_masked]
        out[b, idx] = 1
    return out


def token_ids(shape, vocab, seed=0):
    """Random token ids in [0, vocab), int32."""
    return torch.randint(0, int(vocab), tuple(shape), generator=_gen(seed, "cpu"),
                         dtype=torch.int32)
