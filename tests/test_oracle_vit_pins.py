"""Pins of the oracle's ViT-style block variant (the video VAE decoder block:
affine RMSNorms, per-channel residual scales, per-head RMS q/k norm without
weights, per-head interleaved qkv rows, a rotary embedding on
length-normalized 3-axis coordinates) against closed forms and invariants the
definition fixes."""

import math

import numpy as np

import oracle as O


def test_centered_rope_cache_hand_values_and_symmetry():
    # one frequency per axis (d_a = 2 -> f = 1); grid (1, 1, 2): coordinates
    # t = h = 0 and w = -1/2, +1/2, angles 2 pi c
    cos, sin = O.centered_rope_cache((1, 1, 2), (2, 2, 2), 100.0)
    assert cos.shape == (2, 3)
    assert np.array_equal(cos[:, :2], np.ones((2, 2), np.float32)) and np.array_equal(sin[:, :2], np.zeros((2, 2), np.float32))
    assert cos[0, 2] == np.float32(math.cos(-math.pi)) and cos[1, 2] == np.float32(math.cos(math.pi))
    assert sin[0, 2] == np.float32(math.sin(-math.pi)) and sin[1, 2] == -sin[0, 2]
    # a grid of 5 x 4 x 6: coordinates (2i+1)/n - 1 are symmetric about 0, so
    # cos is even and sin odd under i -> n-1-i on every axis; every |c| < 1
    g = (5, 4, 6)
    dims = (16, 16, 16)
    cos, sin = O.centered_rope_cache(g, dims, 100.0)
    c3, s3 = cos.reshape(*g, 24), sin.reshape(*g, 24)
    assert np.array_equal(c3, c3[::-1, ::-1, ::-1]) and np.array_equal(s3, -s3[::-1, ::-1, ::-1])
    # one hand entry: token (t=1, h=2, w=5), axis h block, frequency j=3: f = 100^(-6/16)
    ang = (2 * math.pi * ((2 * 2 + 1) / 4 - 1)) * (1.0 / 100.0 ** (6 / 16))
    row = (1 * 4 + 2) * 6 + 5
    assert cos[row, 8 + 3] == np.float32(math.cos(ang)) and sin[row, 8 + 3] == np.float32(math.sin(ang))


def _vit_weights(rng, D, F, scale=0.3):
    return {"norm1.weight": 1 + 0.1 * rng.standard_normal(D), "norm2.weight": 1 + 0.1 * rng.standard_normal(D),
            "attn.qkv.weight": rng.standard_normal((3 * D, D)) * scale, "attn.qkv.bias": rng.standard_normal(3 * D) * 0.1,
            "attn.out.weight": rng.standard_normal((D, D)) * scale, "attn.out.bias": rng.standard_normal(D) * 0.1,
            "scale1": rng.standard_normal(D) * 0.5, "scale2": rng.standard_normal(D) * 0.5,
            "ff.w1.weight": rng.standard_normal((2 * F, D)) * scale, "ff.w1.bias": rng.standard_normal(2 * F) * 0.1,
            "ff.w2.weight": rng.standard_normal((D, F)) * scale, "ff.w2.bias": rng.standard_normal(D) * 0.1}


def test_vit_block_closed_form_on_one_token_documents():
    """One-token documents make attention return v; with an identity output
    projection and w1 = [I; 2I], w2 = I the block is, per token,
    x1 = x + s1 (v + b_o), x2 = x1 + s2 silu(h2) 2 h2 with h = RMS(x) g1,
    v_head = h W_v_head^T + b_v_head taken from rows 3 hd h + 2 hd .. 3 hd h + 3 hd
    (the per-head interleaved layout), h2 = RMS(x1) g2.

    Mutations this catches: v read from the rows [2D, 3D) (the [q_all | k_all |
    v_all] layout), the norm weights or the residual scales dropped or swapped,
    the gated halves exchanged."""
    rng = np.random.default_rng(11)
    D, H = 12, 3
    hd = D // H
    w = _vit_weights(rng, D, D)
    w["attn.out.weight"] = np.eye(D)
    w["ff.w1.weight"] = np.vstack([np.eye(D), 2 * np.eye(D)])  # [gate | up] = [h2 | 2 h2]
    w["ff.w1.bias"] = np.zeros(2 * D)
    w["ff.w2.weight"] = np.eye(D)
    w["ff.w2.bias"] = np.zeros(D)
    x = rng.standard_normal((3, D))
    cu = np.array([0, 1, 2, 3])
    cos, sin = np.ones((3, 2)), np.zeros((3, 2))  # one-token documents: the rotation cancels
    got = O.vit_block_forward(x, w, H, 4, 1e-6, cu, cos, sin)
    rms = lambda a: a / np.sqrt((a * a).sum(axis=1, keepdims=True) / D + 1e-6)  # noqa: E731
    h = rms(x) * w["norm1.weight"]
    v = np.empty((3, D))
    for hh in range(H):
        rows = slice(3 * hd * hh + 2 * hd, 3 * hd * hh + 3 * hd)
        v[:, hh * hd:(hh + 1) * hd] = h @ w["attn.qkv.weight"][rows].T + w["attn.qkv.bias"][rows]
    x1 = x + w["scale1"] * (v + w["attn.out.bias"])
    h2 = rms(x1) * w["norm2.weight"]
    want = x1 + w["scale2"] * (h2 / (1 + np.exp(-h2))) * (2 * h2)
    assert np.abs(got - want).max() < 1e-12
    # the concatenated reading of the same weights gives another block
    v_cat = h @ w["attn.qkv.weight"][2 * D:].T + w["attn.qkv.bias"][2 * D:]
    assert np.abs((x + w["scale1"] * (v_cat + w["attn.out.bias"])) - x1).max() > 1e-2


def _two_docs(rng, D, H, rot):
    grid = (2, 2, 3)
    n = 12
    x = rng.standard_normal((2 * n, D))
    cos, sin = O.centered_rope_cache(grid, (rot // 3,) * 3, 100.0)
    cos, sin = np.vstack([cos, cos]), np.vstack([sin, sin])
    return x, np.array([0, n, 2 * n]), cos, sin


def test_vit_qk_norm_makes_the_block_invariant_to_q_and_k_scale():
    """RMS-normalising each head's q and k makes the block independent of the
    scale of the q and k projections; v is not normalised, so scaling the v
    projection (without the MLP) scales the attention sub-layer's update.

    Mutations this catches: the q/k norm dropped, applied to v as well, or
    taken over the whole row instead of each head (then scaling one head's q
    would still be invisible but scaling different heads differently is not)."""
    rng = np.random.default_rng(12)
    D, H, rot = 24, 2, 6
    hd = D // H
    w = _vit_weights(rng, D, 16)
    x, cu, cos, sin = _two_docs(rng, D, H, rot)
    base = O.vit_block_forward(x, w, H, rot, 1e-6, cu, cos, sin)
    w2 = {k: v.copy() for k, v in w.items()}
    for hh, c in ((0, 300.0), (1, 5.0)):  # upward only: the eps term stays negligible
        for part, cc in ((0, c), (1, 7.0 * c)):
            rows = slice(3 * hd * hh + part * hd, 3 * hd * hh + (part + 1) * hd)
            w2["attn.qkv.weight"][rows] *= cc
            w2["attn.qkv.bias"][rows] *= cc
    got = O.vit_block_forward(x, w2, H, rot, 1e-6, cu, cos, sin)
    assert np.abs(got - base).max() < 1e-6 * np.abs(base).max()
    # v scales linearly through the attention sub-layer (MLP switched off)
    w3 = {k: v.copy() for k, v in w.items()}
    w3["scale2"] = np.zeros(D)
    w3["attn.out.bias"] = np.zeros(D)
    a = O.vit_block_forward(x, w3, H, rot, 1e-6, cu, cos, sin) - x
    for hh in range(H):
        rows = slice(3 * hd * hh + 2 * hd, 3 * hd * hh + 3 * hd)
        w3["attn.qkv.weight"][rows] *= 3.0
        w3["attn.qkv.bias"][rows] *= 3.0
    b = O.vit_block_forward(x, w3, H, rot, 1e-6, cu, cos, sin) - x
    assert np.allclose(b, 3.0 * a, rtol=1e-12, atol=1e-12)


def test_vit_block_documents_are_independent():
    rng = np.random.default_rng(13)
    D, H, rot = 24, 2, 6
    w = _vit_weights(rng, D, 16)
    x, cu, cos, sin = _two_docs(rng, D, H, rot)
    packed = O.vit_block_forward(x, w, H, rot, 1e-6, cu, cos, sin)
    alone = O.vit_block_forward(x[12:], w, H, rot, 1e-6, np.array([0, 12]), cos[12:], sin[12:])
    assert np.allclose(packed[12:], alone, rtol=0, atol=1e-12)
    x2 = x.copy()
    x2[3] += 1.0
    moved = O.vit_block_forward(x2, w, H, rot, 1e-6, cu, cos, sin)
    assert np.array_equal(moved[12:], packed[12:]) and not np.allclose(moved[:12], packed[:12])
