"""The ViT-style block variant (the video VAE decoder block) on the same
kernels, through the C ABI, against the oracle's ``vit_block_forward``.

The library runs it as a DiT block of an fp32-stream model whose qkv rows are
staged from the per-head layout, whose q/k are RMS-normalised per head inside
the RoPE kernel, whose rotary table comes from centred coordinates, and whose
modulation is one constant row: shift 0, scale g - 1 (so the modulated norm
is RMSNorm(x) * g exactly: g - 1 is exact in fp32 for g in [0.5, 2]) and gate
= the learned residual scale."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import assert_f32_close
from synthetic.configs import Segment, scaled

pytestmark = pytest.mark.gpu


def _vit_weights(cfg, seed):
    rng = np.random.default_rng(seed)
    D, F = cfg.hidden, cfg.ffn
    f32 = lambda a: np.asarray(a, np.float32)  # noqa: E731
    w = {"norm1.weight": f32(1 + 0.1 * rng.standard_normal(D)), "norm2.weight": f32(1 + 0.1 * rng.standard_normal(D)),
         "scale1": f32(0.5 * rng.standard_normal(D)), "scale2": f32(0.5 * rng.standard_normal(D)),
         "attn.qkv.weight": f32(0.02 * rng.standard_normal((3 * D, D))), "attn.qkv.bias": f32(0.1 * rng.standard_normal(3 * D)),
         "attn.out.weight": f32(0.02 * rng.standard_normal((D, D))), "attn.out.bias": f32(0.1 * rng.standard_normal(D)),
         "ff.w1.weight": f32(0.02 * rng.standard_normal((2 * F, D))), "ff.w1.bias": f32(0.1 * rng.standard_normal(2 * F)),
         "ff.w2.weight": f32(0.02 * rng.standard_normal((D, F))), "ff.w2.bias": f32(0.1 * rng.standard_normal(D))}
    return w


def _as_dit(cfg, w):
    """The DiT weight contract's names for the ViT block's tensors (AdaLN
    linears zero: the modulation row is passed in directly)."""
    D = cfg.hidden
    return {"blocks.0.adaln.0.weight": np.zeros((6 * D, cfg.cond_dim), np.float32),
            "blocks.0.adaln.0.bias": np.zeros(6 * D, np.float32),
            "blocks.0.attn.qkv.weight": w["attn.qkv.weight"], "blocks.0.attn.qkv.bias": w["attn.qkv.bias"],
            "blocks.0.attn.out.weight": w["attn.out.weight"], "blocks.0.attn.out.bias": w["attn.out.bias"],
            "blocks.0.mlp.in.weight": w["ff.w1.weight"], "blocks.0.mlp.in.bias": w["ff.w1.bias"],
            "blocks.0.mlp.out.weight": w["ff.w2.weight"], "blocks.0.mlp.out.bias": w["ff.w2.bias"]}


def _mod_row(cfg, w):
    D = cfg.hidden
    row = np.zeros((1, 6, D), np.float32)
    for k, (g, s) in enumerate(((w["norm1.weight"], w["scale1"]), (w["norm2.weight"], w["scale2"]))):
        gm1 = (g - np.float32(1)).astype(np.float32)
        assert np.array_equal(np.float32(1) + gm1, g)  # exact: the modulated norm is RMSNorm(x) * g
        row[0, 3 * k + 1] = gm1
        row[0, 3 * k + 2] = s
    return row


@pytest.mark.parametrize("name", ["vit3d", "vit3d_ragged_docs"])
def test_vit_block_matches_oracle(name):
    import harness
    from video_audio_gen_amd import dit
    cfg = S.get_config("vit")
    if name == "vit3d_ragged_docs":  # single-token and odd documents beside a larger one
        cfg = scaled(cfg, segments=(Segment(0, (1, 1, 1), 0), Segment(0, (3, 5, 7), 0), Segment(0, (1, 2, 3), 0)))
    print(f"vit block {name}: {cfg.n_tokens} tokens, hidden {cfg.hidden}", flush=True)
    w = _vit_weights(cfg, 61)
    m = dit.Model(cfg)
    dit.dit_stage_weights(m, _as_dit(cfg, w))
    dit.dit_stage_finalize(m)
    batch = harness.make_batch(m, cfg)
    ws = dit.workspace(batch)
    x = np.random.default_rng(62).standard_normal((cfg.n_tokens, cfg.hidden)).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    mod = torch.from_numpy(_mod_row(cfg, w)).cuda()
    dit.dit_block_forward(m, 0, xd, mod, batch, ws)
    torch.cuda.synchronize()
    got = xd.cpu().numpy().astype(np.float64)
    cos, sin = O.rope_cache(cfg)
    lay = O.pack_layout(cfg)
    ref = O.vit_block_forward(x.astype(np.float64), {k: v.astype(np.float64) for k, v in w.items()}, cfg.n_heads,
                              cfg.rot_dim, cfg.norm_eps, lay["cu_seqlens"], cos, sin)
    err = np.abs(got - ref)
    print(f"vit block {name}: max|d| {err.max():.3e}, worst err/bound {(err / (1e-6 + 1e-5 * np.abs(ref))).max():.3f}")
    assert_f32_close(got, ref, what=f"vit block {name}")
    c = dit.dit_counters()
    assert c["rope_split"] > 0 and c["attention_f32"] > 0


def test_vit_block_per_head_rows_are_not_the_concatenated_reading():
    """The same weights staged as a [q_all | k_all | v_all] model give another
    block: the layout flag is what makes the per-head checkpoint correct."""
    import harness
    from video_audio_gen_amd import dit
    cfg = scaled(S.get_config("vit"), segments=(Segment(0, (1, 4, 6), 0),))
    w = _vit_weights(cfg, 63)
    outs = []
    for c in (cfg, scaled(cfg, qkv_layout="concat")):
        m = dit.Model(c)
        dit.dit_stage_weights(m, _as_dit(c, w))
        dit.dit_stage_finalize(m)
        batch = harness.make_batch(m, c)
        ws = dit.workspace(batch)
        xd = torch.from_numpy(np.random.default_rng(64).standard_normal((c.n_tokens, c.hidden)).astype(np.float32)).cuda()
        dit.dit_block_forward(m, 0, xd, torch.from_numpy(_mod_row(c, w)).cuda(), batch, ws)
        torch.cuda.synchronize()
        outs.append(xd.cpu().numpy())
    assert np.abs(outs[0] - outs[1]).max() > 1e-2
