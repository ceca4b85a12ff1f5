"""Pins for the gradient oracle (oracle.wall_attn_bwd): checks against facts
fixed outside it.

  * Central finite differences of the forward oracle -- the Wall Attention
    README's own test of the gradients of g and g_scalar ("Tests") -- for
    every element of every input (q, k, v, g, g_scalar, sink_bias), with a
    window and with packed sequences.  The forward oracle is pinned in
    test_oracle_pins.py.
  * torch autograd through a library routine: exp(P_i - P_j) = e^{P_i}
    e^{-P_j}, so the forward is torch's scaled_dot_product_attention (CPU,
    fp64) on (q e^P, k e^-P) with P = torch.cumsum(g), the gate as an additive
    mask Gs_i - Gs_j and the window as -inf outside the band; autograd through
    cumsum, exp, repeat_interleave and SDPA gives dq, dk, dv, dg, dg_scalar.
A dropped key-side term of dP, a wrong sign, a missing GQA sum or a forward
(instead of reverse) running sum fails both.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

f64 = torch.float64


def _rand(shape, seed, scale=1.0):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * scale


def _loss(x, dO, **kw):
    o = oracle.wall_attn(x["q"], x["k"], x["v"], x["g"], g_scalar=x.get("g_scalar"),
                         sink_bias=x.get("sink_bias"), **kw)
    return float((o * dO.numpy().astype(np.float64)).sum())


def _fd_check(x, dO, grads, keys, **kw):
    eps = 2.0 ** -10  # exact in float32 for the |x| < 16 used here
    for key in keys:
        base = x[key].clone()
        flat = base.reshape(-1)
        num = np.zeros(flat.numel())
        for e in range(flat.numel()):
            xp = dict(x)
            t = flat.clone()
            t[e] += eps
            xp[key] = t.reshape(base.shape)
            lp = _loss(xp, dO, **kw)
            t[e] -= 2 * eps
            xp[key] = t.reshape(base.shape)
            lm = _loss(xp, dO, **kw)
            num[e] = (lp - lm) / (2 * eps)
        ana = grads["d" + key if key != "sink_bias" else "dsink"].reshape(-1)
        if key == "g_scalar":
            ana = grads["dg_scalar"].reshape(-1)
        np.testing.assert_allclose(ana, num, rtol=1e-5, atol=2e-7, err_msg=key)


@pytest.mark.parametrize("window", [None, 5])
def test_gradients_match_central_differences(window):
    B, T, HQ, H, K, V = 1, 9, 2, 1, 3, 2
    x = dict(q=_rand((B, T, HQ, K), 1), k=_rand((B, T, H, K), 2), v=_rand((B, T, H, V), 3),
             g=_rand((B, T, HQ, K), 4, 0.3), g_scalar=_rand((B, T, HQ), 5, 0.2),
             sink_bias=_rand((HQ,), 6))
    dO = _rand((B, T, HQ, V), 7)
    grads = oracle.wall_attn_bwd(x["q"], x["k"], x["v"], x["g"], dO, g_scalar=x["g_scalar"],
                                 sink_bias=x["sink_bias"], window_size=window)
    _fd_check(x, dO, grads, ["q", "k", "v", "g", "g_scalar", "sink_bias"], window_size=window)


def test_gradients_match_central_differences_varlen_gqa():
    lens = [4, 1, 6]
    T, HQ, H, K, V = sum(lens), 4, 2, 2, 3
    cu = torch.tensor([0, 4, 5, 11], dtype=torch.int32)
    x = dict(q=_rand((1, T, HQ, K), 11), k=_rand((1, T, H, K), 12), v=_rand((1, T, H, V), 13),
             g=_rand((1, T, HQ, K), 14, 0.3), g_scalar=_rand((1, T, HQ), 15, 0.2))
    dO = _rand((1, T, HQ, V), 17)
    grads = oracle.wall_attn_bwd(x["q"], x["k"], x["v"], x["g"], dO, g_scalar=x["g_scalar"],
                                 cu_seqlens=cu, window_size=3)
    _fd_check(x, dO, grads, ["q", "k", "v", "g", "g_scalar"], cu_seqlens=cu, window_size=3)


@pytest.mark.parametrize("window", [None, 6])
def test_gradients_match_autograd_through_sdpa(window):
    B, T, HQ, H, K, V = 2, 23, 4, 2, 8, 5
    q, k, v = _rand((B, T, HQ, K), 21), _rand((B, T, H, K), 22), _rand((B, T, H, V), 23)
    g, gs = _rand((B, T, HQ, K), 24, 0.2), _rand((B, T, HQ), 25, 0.2)
    dO = _rand((B, T, HQ, V), 26)
    scale = 0.41
    ref = oracle.wall_attn_bwd(q, k, v, g, dO, scale=scale, g_scalar=gs, window_size=window)
    tq, tk, tv, tg, tgs = (t.to(f64).requires_grad_() for t in (q, k, v, g, gs))
    P = torch.cumsum(tg, dim=1)
    G = torch.cumsum(tgs, dim=1)                                   # [B,T,HQ]
    qs = (tq * torch.exp(P)).transpose(1, 2)
    ks = (tk.repeat_interleave(HQ // H, dim=2) * torch.exp(-P)).transpose(1, 2)
    vs = tv.repeat_interleave(HQ // H, dim=2).transpose(1, 2)
    i = torch.arange(T)
    d = i[:, None] - i[None, :]
    allowed = (d >= 0) & (d < (window if window else T + 1))
    bias = G.transpose(1, 2)[..., :, None] - G.transpose(1, 2)[..., None, :]
    mask = bias.masked_fill(~allowed, float("-inf"))
    o = F.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=scale).transpose(1, 2)
    o.backward(dO.to(f64))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dg", tg), ("dg_scalar", tgs)):
        np.testing.assert_allclose(ref[name], t.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)
