"""CPU checks of the seeded inputs themselves: properties that GPU tests rely on
to reach a code path (no GPU, no library)."""
import math

import numpy as np
import torch

from exact_attention_channel_amd import workloads as W


def _anchor_gaps(x, chunk=64, qtile=128):
    """Largest (query-tile anchor - key-chunk anchor) over all visible pairs, per
    channel, in log2 units.  Anchors: the integer nearest to the running sum of
    g (log2 units) at the chunk's last token; a query tile's anchor is its first
    chunk's."""
    g = x["g"].float().numpy()[0]                       # [T, HQ, K]
    P = np.cumsum(g.astype(np.float64), axis=0) / math.log(2)
    L = P.shape[0]
    nch = (L + chunk - 1) // chunk
    R = np.stack([np.rint(P[min(chunk * c + chunk - 1, L - 1)]) for c in range(nch)])
    best = -np.inf
    for I in range((L + qtile - 1) // qtile):
        RQ = R[min(2 * I, nch - 1)]
        best = max(best, float((RQ[None] - R[:min(2 * I + 2, nch)]).max()))
    return best


def test_rising_channel_inputs_reach_rebalancing():
    """The rising-channel GPU cases need an anchor gap above 8 log2 units (the
    kernel's rebalancing threshold) while the rising channel adds nothing to any
    score (its k is zero)."""
    c = W.Prefill("rise", 2, 256, 4, 2, 64, 64, torch.bfloat16, rise_ch0_log2=0.1, seed=24)
    x = W.make_prefill(c)
    gap = _anchor_gaps(x)
    assert 8 < gap <= 16, gap
    assert float(x["k"][..., 0].abs().max()) == 0.0


def test_default_workloads_stay_below_rebalancing():
    """The benchmark workload never rebalances (its decay sums fall), so its
    timing is the common path's."""
    x = W.make_prefill(W.PREFILL_T8192_BF16)
    assert _anchor_gaps(x) <= 8
