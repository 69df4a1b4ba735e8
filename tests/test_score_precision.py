"""The precision the compressed kernel needs for the block scores (CPU only).

The kernel keeps the block means of K scaled by softmax_scale * log2(e) and
rounded to bf16 (the high part), plus the bf16 rounding remainder (the low
part). Queries that see at least 512 blocks score them from the high part
alone. These tests model that arithmetic in float64 on the benchmark's
input distribution (i.i.d. N(0, 1) bf16 tokens, 64-token means, 16 query
heads of dimension 128 per KV group) and check the bound it relies on: the
head-summed probabilities move by much less than half of the 1e-4 gap below
which the selection may legitimately differ from the oracle's, so no row
with a larger gap can change its selection. At 64 visible blocks the high
part alone would not be enough, which is why the low part stays there.
"""

import numpy as np
import pytest

D, HG, BLOCK = 128, 16, 64
SL2 = np.log2(np.e) / np.sqrt(D)


def bf16(x):
    """Round-to-nearest-even to bf16, returned as float64."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def scores(q, kc):
    """Head sums of the softmax probabilities over the blocks (log2 logits q . kc)."""
    s = q @ kc.T
    p = np.exp2(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)).sum(axis=0)


def max_score_error(n_blocks, trials, use_low, seed):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for _ in range(trials):
        toks = bf16(rng.standard_normal((n_blocks, BLOCK, D)).astype(np.float32))
        mean = toks.mean(axis=1) * SL2           # exact scaled means (the oracle's)
        hi = bf16(mean)
        kc = hi + bf16(mean - hi) if use_low else hi
        q = bf16(rng.standard_normal((HG, D)).astype(np.float32))
        worst = max(worst, float(np.abs(scores(q, kc) - scores(q, mean)).max()))
    return worst


@pytest.mark.parametrize("n_blocks", [512, 1023])
def test_high_part_alone_keeps_scores_far_inside_the_tie_band(n_blocks):
    err = max_score_error(n_blocks, trials=24, use_low=False, seed=n_blocks)
    # a flip needs two scores to move by half the 1e-4 gap together
    assert err < 2.5e-5, err


def test_low_part_is_needed_at_few_blocks_and_enough_there():
    assert max_score_error(64, trials=40, use_low=False, seed=1) > 2.5e-5
    assert max_score_error(64, trials=40, use_low=True, seed=1) < 1e-6
