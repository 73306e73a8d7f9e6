"""Pins of the CPU oracle against what the mathematics and the pages fix.

Each test checks an oracle function against something other than itself: a
closed form, a hand-derived value, an invariant, brute force on a tiny input,
or a library routine for a special case.  They are chosen so that a plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a wrong
half of a merged projection, the wrong modulation row) fails at least one.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from synthetic.configs import CondRow, DitConfig, Modality, Segment, scaled


# ----------------------------------------------------------------------------- rounding

def test_round_bf16_ties_and_library():
    one = 1.0
    ulp = 2.0 ** -7
    x = np.array([one, one + ulp / 2, one + 1.5 * ulp, one + 0.75 * ulp, -(one + ulp / 2), 3.0e-3])
    got = O.round_bf16(x)
    # ties go to the even mantissa; 0.75 ulp rounds up
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == one + 2 * ulp and got[3] == one + ulp
    assert got[4] == -1.0
    # against torch's float32 -> bfloat16 conversion (round to nearest even)
    r = np.random.default_rng(0).standard_normal(20000).astype(np.float32) * 3
    ref = torch.from_numpy(r).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(r.astype(np.float64)), ref)


# ----------------------------------------------------------------------------- layout and positions

@pytest.mark.parametrize("name,cu", [
    ("c1", [0, 64, 160]), ("c2", [0, 86, 172]), ("c3", [0, 24576, 26624]),
    ("c4", [0, 8192, 9216, 17408, 18432]), ("c5", [0, 16384, 18432])])
def test_pack_layout_hand_offsets(name, cu):
    cfg = S.get_config(name)
    lay = O.pack_layout(cfg)
    assert lay["cu_seqlens"].tolist() == cu
    counts = np.bincount(lay["cond_idx"], minlength=cfg.n_cond)
    for i, s in enumerate(cfg.segments):
        assert (lay["cond_idx"][cu[i]:cu[i + 1]] == s.cond_row).all()
        assert (lay["doc_id"][cu[i]:cu[i + 1]] == i).all()
    assert counts.sum() == cu[-1]


def test_token_positions_raster_order():
    pos = O.token_positions(S.get_config("c1"))
    # second document (grid 4x4x6) starts at row 64; its token 37 is t=1, h=2, w=1
    assert pos[64 + 37] == [1, 2, 1]
    assert pos[0] == [0, 0, 0] and pos[63] == [3, 3, 3] and pos[64] == [0, 0, 0]
    assert pos[159] == [3, 3, 5]


def test_rope_inv_freq_closed_form():
    f = O.rope_inv_freq(8, 10000.0)
    assert np.allclose(f, [1.0, 0.1, 0.01, 0.001], rtol=1e-15, atol=0)
    g = O.rope_inv_freq(128, 10000.0)
    assert len(g) == 64 and g[0] == 1.0 and abs(g[32] - 0.01) < 1e-16


def test_rope_cache_origin_and_hand_row():
    cfg = S.get_config("c1")
    cos, sin = O.rope_cache(cfg)
    for r in (0, 64):  # the first token of each document sits at the origin
        assert (cos[r] == 1.0).all() and (sin[r] == 0.0).all()
    # row 64+37 = (t, h, w) = (1, 2, 1); axes 8/12/12 -> 4/6/6 frequencies
    r = 64 + 37
    ang = [1 * 10000.0 ** (-2 * j / 8) for j in range(4)] + \
          [2 * 10000.0 ** (-2 * j / 12) for j in range(6)] + \
          [1 * 10000.0 ** (-2 * j / 12) for j in range(6)]
    assert np.allclose(cos[r], np.cos(ang), rtol=0, atol=1e-7)
    assert np.allclose(sin[r], np.sin(ang), rtol=0, atol=1e-7)


# ----------------------------------------------------------------------------- RoPE

def _fp64_cache(pos, inv):
    ang = np.outer(pos, inv)
    return np.cos(ang), np.sin(ang)


def test_rope_rotate_half_direction_and_pairing():
    # rotate_half(x) = [-x2, x1]: e_0 at angle pi/2 goes to e_{rot/2}; e_{rot/2} to -e_0
    x = np.zeros((1, 1, 8))
    x[0, 0, 0] = 1.0
    c = np.array([[0.0, 1.0, 1.0, 1.0]])
    s = np.array([[1.0, 0.0, 0.0, 0.0]])
    out = O.apply_rope(x, c, s, 8)
    assert np.allclose(out[0, 0], [0, 0, 0, 0, 1, 0, 0, 0], atol=1e-15)
    x = np.zeros((1, 1, 8))
    x[0, 0, 4] = 1.0
    out = O.apply_rope(x, c, s, 8)
    assert np.allclose(out[0, 0], [-1, 0, 0, 0, 0, 0, 0, 0], atol=1e-15)


def test_rope_norm_composition_passthrough_relative():
    rng = np.random.default_rng(1)
    hd, rot = 16, 8
    inv = np.array(O.rope_inv_freq(rot, 10000.0))
    x = rng.standard_normal((5, 3, hd))
    p = np.array([0, 1, 7, 33, 1000], float)
    c, s = _fp64_cache(p, inv)
    y = O.apply_rope(x, c, s, rot)
    # norm preserved per head; dims >= rot untouched bit for bit
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    assert np.array_equal(y[..., rot:], x[..., rot:])
    # rope(rope(x, p), p2) == rope(x, p + p2)
    p2 = np.array([3, 4, 5, 6, 7], float)
    c2, s2 = _fp64_cache(p2, inv)
    c3, s3 = _fp64_cache(p + p2, inv)
    assert np.allclose(O.apply_rope(y, c2, s2, rot), O.apply_rope(x, c3, s3, rot), atol=1e-12)
    # relative position: q(p+d) . k(p'+d) == q(p) . k(p')
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    def dot(pq, pk):
        cq, sq = _fp64_cache(np.array([pq], float), inv)
        ck, sk = _fp64_cache(np.array([pk], float), inv)
        return float((O.apply_rope(q, cq, sq, rot) * O.apply_rope(k, ck, sk, rot)).sum())
    assert abs(dot(3, 10) - dot(53, 60)) < 1e-12
    assert abs(dot(3, 10) - dot(10, 3)) > 1e-6  # not symmetric: the sign of the offset matters


# ----------------------------------------------------------------------------- norm and modulate

def test_norms_closed_forms():
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    eps = 1e-6
    assert np.allclose(O.norm(x, "rms", eps), x / math.sqrt(7.5 + eps), rtol=1e-15)
    assert np.allclose(O.norm(x, "layer", eps), (x - 2.5) / math.sqrt(1.25 + eps), rtol=1e-15)
    c = np.full((1, 64), -3.0)
    assert np.allclose(O.norm(c, "rms", eps), -3.0 / math.sqrt(9.0 + eps), rtol=1e-15)
    assert np.allclose(O.norm(c, "layer", eps), 0.0, atol=1e-12)
    y = O.norm(np.random.default_rng(2).standard_normal((3, 256)) * 5 + 2, "layer", eps)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-13)
    assert np.allclose(y.var(axis=1), 1, atol=1e-6)


def test_modulate_forms():
    y = np.array([1.0, -2.0])
    assert np.array_equal(O.modulate(y, np.zeros(2), np.zeros(2)), y)
    assert np.array_equal(O.modulate(y, np.array([0.5, 0.5]), np.ones(2)), np.array([2.5, -3.5]))


# ----------------------------------------------------------------------------- attention

def test_attention_matches_dense_masked_bruteforce():
    rng = np.random.default_rng(3)
    cu = np.array([0, 1, 9, 26, 40], np.int32)  # includes a one-token document
    q, k, v = (rng.standard_normal((40, 3, 8)) for _ in range(3))
    a = O.attention_varlen(q, k, v, cu)
    b = O.attention_dense_masked(q, k, v, cu)
    assert np.allclose(a, b, atol=1e-13)
    assert np.allclose(a[0], v[0], atol=0)  # a one-token document returns its value


def test_attention_scale_and_identical_keys():
    # scores 2 and 0 scaled by 1/sqrt(4): p = softmax([1, 0]) -> o = e/(1+e) for v = (1, 0)
    q = np.zeros((2, 1, 4)); q[:, 0, 0] = 2.0
    k = np.zeros((2, 1, 4)); k[0, 0, 0] = 1.0
    v = np.zeros((2, 1, 4)); v[0, 0, 0] = 1.0
    o = O.attention_varlen(q, k, v, np.array([0, 2]))
    assert abs(o[0, 0, 0] - math.e / (1 + math.e)) < 1e-15
    # identical keys: uniform weights, the output is the mean of the values
    rng = np.random.default_rng(4)
    q = rng.standard_normal((6, 2, 4)); k = np.tile(rng.standard_normal((1, 2, 4)), (6, 1, 1))
    v = rng.standard_normal((6, 2, 4))
    o = O.attention_varlen(q, k, v, np.array([0, 6]))
    assert np.allclose(o, v.mean(axis=0, keepdims=True), atol=1e-14)


def test_attention_segmentation_bit_identical():
    rng = np.random.default_rng(5)
    cu = np.array([0, 20, 50], np.int32)
    q, k, v = (rng.standard_normal((50, 2, 8)) for _ in range(3))
    a = O.attention_varlen(q, k, v, cu)
    k2 = k.copy(); v2 = v.copy()
    k2[30] += 1.0; v2[40] -= 2.0  # perturb the second document only
    b = O.attention_varlen(q, k2, v2, cu)
    assert np.array_equal(a[:20], b[:20])
    assert not np.allclose(a[20:], b[20:])
    alone = O.attention_varlen(q[20:], k[20:], v[20:], np.array([0, 30]))
    assert np.array_equal(alone, a[20:])


# ----------------------------------------------------------------------------- MLP pieces

def test_silu_and_merged_halves():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    h = 1e-6
    assert abs((O.silu(np.array([h])) - O.silu(np.array([-h])))[0] / (2 * h) - 0.5) < 1e-9
    u = np.array([[1.0, 2.0]])  # F = 1
    assert abs(O.split_mlp(u, "gate_up", 1)[0, 0] - 2.0 * O.silu(np.array([1.0]))[0]) < 1e-15
    assert abs(O.split_mlp(u, "value_gate", 1)[0, 0] - 1.0 * O.silu(np.array([2.0]))[0]) < 1e-15


def test_linear_identity_and_hand_product():
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert np.array_equal(O.linear(x, np.eye(2), np.zeros(2)), x)
    W = np.array([[1.0, 0.0], [1.0, -1.0], [0.5, 2.0]])  # [out=3, in=2]
    assert np.array_equal(O.linear(x, W, np.array([0.0, 1.0, 0.0])),
                          np.array([[1.0, 0.0, 4.5], [3.0, 0.0, 9.5]]))


# ----------------------------------------------------------------------------- AdaLN table and conditioning

def _tiny_cfg(**kw):
    base = dict(name="tiny", key_id=99, model_id=99, n_blocks=1, hidden=8, n_heads=2, head_dim=4, ffn=8,
                norm="rms", norm_eps=1e-6, mlp="gate_up", rot_dim=4, theta=10000.0, stream="f32",
                cond_kind="timestep", cond_dim=4,
                modalities=(Modality("a", "none", 0, (1, 1, 1), (4,)), Modality("b", "none", 0, (1, 1, 1), (4,))),
                segments=(Segment(0, (1,), 0), Segment(1, (1,), 1), Segment(0, (1,), 0)),
                cond_rows=(CondRow(0, 0), CondRow(1, 0)), n_requests=1, io=False)
    base.update(kw)
    return DitConfig(**base)


def test_adaln_table_layout_and_modality_choice():
    cfg = _tiny_cfg()
    D, dt = cfg.hidden, cfg.cond_dim
    rng = np.random.default_rng(6)
    bw = {"blocks.0.adaln.0.weight": rng.standard_normal((6 * D, dt)),
          "blocks.0.adaln.0.bias": rng.standard_normal(6 * D),
          "blocks.0.adaln.1.weight": rng.standard_normal((6 * D, dt)),
          "blocks.0.adaln.1.bias": rng.standard_normal(6 * D)}
    emb = np.zeros((2, dt)); emb[0, 2] = 1.0; emb[1, 3] = 1.0
    mod = O.adaln_table(cfg, bw, 0, emb, "fp64")
    # row 0 uses modality 0's linear: column 2 of W plus bias, split into 6 chunks of D
    want0 = (bw["blocks.0.adaln.0.weight"][:, 2] + bw["blocks.0.adaln.0.bias"]).reshape(6, D)
    want1 = (bw["blocks.0.adaln.1.weight"][:, 3] + bw["blocks.0.adaln.1.bias"]).reshape(6, D)
    assert np.array_equal(mod[0], want0) and np.array_equal(mod[1], want1)
    assert np.array_equal(mod[0, 2], bw["blocks.0.adaln.0.weight"][2 * D:3 * D, 2] + bw["blocks.0.adaln.0.bias"][2 * D:3 * D])


def test_timestep_embedding_closed_form():
    e0 = O.timestep_embedding(0.0, 8)
    assert np.array_equal(e0, np.array([1, 1, 1, 1, 0, 0, 0, 0], np.float32))
    e1 = O.timestep_embedding(1.0, 4)  # f = [1, 10000^-1/2 = 0.01]
    assert np.allclose(e1, [math.cos(1), math.cos(0.01), math.sin(1), math.sin(0.01)], atol=1e-7)


# ----------------------------------------------------------------------------- block wiring

def _identity_block(cfg):
    D, F = cfg.hidden, cfg.ffn
    assert F == D
    z = lambda *s: np.zeros(s)  # noqa: E731
    qkv = np.zeros((3 * D, D)); qkv[2 * D:] = np.eye(D)  # v = h, q = k = 0
    w_in = np.vstack([np.eye(D), np.eye(D)])              # u = [h2 | h2]
    return {"blocks.0.attn.qkv.weight": qkv, "blocks.0.attn.qkv.bias": z(3 * D),
            "blocks.0.attn.out.weight": np.eye(D), "blocks.0.attn.out.bias": z(D),
            "blocks.0.mlp.in.weight": w_in, "blocks.0.mlp.in.bias": z(2 * F),
            "blocks.0.mlp.out.weight": np.eye(D), "blocks.0.mlp.out.bias": z(D)}


def test_block_closed_form_on_single_token_documents():
    # One-token documents make attention return v, so with identity projections
    # x1 = x + g_msa * h and x2 = x1 + g_mlp * silu(h2) * h2 in closed form.
    cfg = _tiny_cfg()
    rng = np.random.default_rng(7)
    D = cfg.hidden
    x = rng.standard_normal((3, D))
    mod = rng.standard_normal((2, 6, D)) * 0.5
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    out = O.block_forward(cfg, x, mod, _identity_block(cfg), 0, lay, cos, sin, "fp64")
    ci = lay["cond_idx"]
    m = mod[ci]
    rms = lambda a: a / np.sqrt((a * a).mean(axis=1, keepdims=True) + cfg.norm_eps)  # noqa: E731
    h = rms(x) * (1 + m[:, 1]) + m[:, 0]
    x1 = x + m[:, 2] * h
    h2 = rms(x1) * (1 + m[:, 4]) + m[:, 3]
    x2 = x1 + m[:, 5] * (h2 / (1 + np.exp(-h2))) * h2
    assert np.allclose(out, x2, atol=1e-13)


@pytest.mark.parametrize("mode", ["fp64", "bf16"])
def test_zero_gate_block_is_identity(mode):
    cfg = scaled(S.get_config("c1"), stream="bf16" if mode == "bf16" else "f32")
    w = S.block_weights(cfg, 0)
    inp = S.inputs(cfg)
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    mod = np.random.default_rng(8).standard_normal((1, 6, cfg.hidden))
    mod[:, 2] = 0.0
    mod[:, 5] = 0.0
    x = O.round_f32(inp["x"].astype(np.float64))
    out = O.block_forward(cfg, x, mod, w, 0, lay, cos, sin, mode)
    assert np.array_equal(out, x)


def test_packed_equals_alone_block():
    cfg = S.get_config("c1")
    w = S.block_weights(cfg, 0)
    x = S.inputs(cfg)["x"].astype(np.float64)
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    mod = np.random.default_rng(9).standard_normal((1, 6, cfg.hidden)) * 0.3
    packed = O.block_forward(cfg, x, mod, w, 0, lay, cos, sin, "fp64")
    for i, seg in enumerate(cfg.segments):
        a, b = int(lay["cu_seqlens"][i]), int(lay["cu_seqlens"][i + 1])
        one = scaled(cfg, segments=(seg,))
        lay1 = O.pack_layout(one)
        c1, s1 = O.rope_cache(one)
        alone = O.block_forward(one, x[a:b], mod, w, 0, lay1, c1, s1, "fp64")
        assert np.allclose(alone, packed[a:b], rtol=0, atol=1e-12)


def test_swapped_mlp_halves_change_the_block():
    # a [value | gate] model read as [gate | up] must not pass (mutation check)
    cfg = scaled(S.get_config("c1"), mlp="value_gate")
    w = S.block_weights(cfg, 0)
    x = S.inputs(cfg)["x"].astype(np.float64)
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    mod = np.random.default_rng(10).standard_normal((1, 6, cfg.hidden)) * 0.3
    a = O.block_forward(cfg, x, mod, w, 0, lay, cos, sin, "fp64")
    b = O.block_forward(scaled(cfg, mlp="gate_up"), x, mod, w, 0, lay, cos, sin, "fp64")
    assert np.abs(a - b).max() > 1e-3


# ----------------------------------------------------------------------------- patch islands

def test_patchify_hand_permutation_and_round_trip():
    mod = Modality("v", "patch3d", 2, (1, 2, 2), (2, 2, 2))
    lat = np.arange(16, dtype=np.float64).reshape(2, 1, 4, 2)  # C=2, T=1, H=2*2, W=1*2
    tok = O.patchify(lat, mod)
    assert tok.tolist() == [[0, 8, 1, 9, 2, 10, 3, 11], [4, 12, 5, 13, 6, 14, 7, 15]]
    assert np.array_equal(O.unpatchify(tok, mod, (1, 2, 1)), lat)
    big = np.random.default_rng(11).standard_normal((16, 3, 8, 12))
    vm = Modality("v", "patch3d", 16, (1, 2, 2), (2, 2, 2))
    assert np.array_equal(O.unpatchify(O.patchify(big, vm), vm, (3, 4, 6)), big)
    am = Modality("a", "channel_major", 32, (1, 1, 1), (4,))
    al = np.random.default_rng(12).standard_normal((32, 7))
    assert np.array_equal(O.patchify(al, am), al.T)
    assert np.array_equal(O.unpatchify(O.patchify(al, am), am, (7,)), al)


# ----------------------------------------------------------------------------- schedule and Euler

def test_sigma_schedule_closed_forms():
    s = O.sigma_schedule(12.0, 50)
    assert s[0] == 1.0 and s[-1] == 0.0 and (np.diff(s) < 0).all()
    assert abs(s[25] - 6.0 / 6.5) < 1e-15
    lin = O.sigma_schedule(1.0, 10)
    assert np.allclose(lin, 1 - np.arange(11) / 10, atol=1e-16)


def test_euler_telescopes_and_eta0_forms_agree():
    sig = O.sigma_schedule(3.0, 50)
    dt = O.sigma_dt(sig)
    x0 = np.random.default_rng(13).standard_normal(1000).astype(np.float32)
    v = np.random.default_rng(14).standard_normal(1000).astype(np.float32)
    x = x0.copy()
    for i in range(50):
        x = O.euler_step(x, v, dt[i])
    assert np.abs(x.astype(np.float64) - (x0.astype(np.float64) - v)).max() < 2e-5
    # ancestral eta=0 with x0_hat = x - sigma v: (s'/s) x + (1 - s'/s) x0_hat == x + (s' - s) v
    s, s2 = sig[10], sig[11]
    xx = x0.astype(np.float64)
    anc = (s2 / s) * xx + (1 - s2 / s) * (xx - s * v)
    assert np.allclose(anc, xx + (s2 - s) * v, atol=1e-14)


# ----------------------------------------------------------------------------- whole forward

def test_cfg_branches_differ_and_stay_finite():
    # the music configuration at reduced depth: two CFG branches on one latent
    cfg = scaled(S.get_config("c2"), n_blocks=1, hidden=256, n_heads=2, ffn=512)
    isl = S.island_weights(cfg)
    out = O.forward(cfg, lambda b: S.block_weights(cfg, b), isl, S.inputs(cfg))
    a, b = out["latent.0"], out["latent.1"]
    assert a.shape == (128, 86) and np.isfinite(a).all() and np.isfinite(b).all()
    assert np.abs(a - b).max() > 1e-3


def test_timestep_forward_packed_equals_alone():
    cfg = scaled(S.get_config("c4"), n_blocks=1, hidden=256, n_heads=2, ffn=256,
                 segments=(Segment(0, (1, 2, 4), 0), Segment(1, (6,), 1)),
                 cond_rows=(CondRow(0, 0), CondRow(1, 0)), n_requests=1)
    isl = S.island_weights(cfg)
    inp = S.inputs(cfg)
    W = lambda b: S.block_weights(cfg, b)  # noqa: E731
    packed = O.forward(cfg, W, isl, inp)
    for i, seg in enumerate(cfg.segments):
        one = scaled(cfg, segments=(Segment(seg.modality, seg.grid, seg.cond_row),))
        alone = O.forward(one, W, isl, {"latent.0": inp[f"latent.{i}"], "t": inp["t"]},
                          t_rows=[float(inp["t"][0])] * 2)
        assert np.allclose(alone["latent.0"], packed[f"latent.{i}"], rtol=0, atol=1e-12)


def test_linear_fp32_accumulation_is_the_float32_product():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((7, 300)).astype(np.float32)
    W = rng.standard_normal((5, 300)).astype(np.float32)
    b = rng.standard_normal(5)
    got = O.linear(x, W, b, accum="fp32")
    assert np.array_equal(got, (x @ W.T).astype(np.float64) + b)
    assert 0 < np.abs(got - O.linear(x, W, b)).max() < 1e-4


def test_denoise_loop_constant_velocity_telescopes():
    # no blocks and a zero output projection: v = the output bias everywhere,
    # so n Euler steps move each latent by sum(dt) * bias = -bias (sigma 1 -> 0)
    cfg = scaled(S.get_config("c5"), n_blocks=0, hidden=256, n_heads=2, ffn=512, denoise_steps=6,
                 segments=(Segment(0, (1, 2, 2), 0), Segment(1, (5,), 1)))
    isl = S.island_weights(cfg)
    bias = {}
    for m in range(cfg.n_mod):
        isl[f"out.{m}.weight"][:] = 0.0
        bias[m] = np.random.default_rng(20 + m).standard_normal(isl[f"out.{m}.bias"].shape).astype(np.float32)
        isl[f"out.{m}.bias"][:] = bias[m]
    lat0 = S.inputs(cfg)
    out = O.denoise_loop(cfg, lambda b: {}, isl, lat0, 6)
    for j, seg in enumerate(cfg.segments):
        mod = cfg.modalities[seg.modality]
        v = O.unpatchify(np.tile(bias[seg.modality], (seg.n_tokens, 1)), mod, seg.grid)
        want = lat0[f"latent.{j}"].astype(np.float64) - v
        assert np.abs(out[f"latent.{j}"] - want).max() < 1e-5
    # and a different shift per modality gives different intermediate sigmas
    t6, _ = O.denoise_step_conditions(cfg, 3)
    assert t6[0] != t6[1]


# ----------------------------------------------------------------------------- guided (CFG) loop

def test_cfg_combine_hand_values():
    vc = np.array([3.0, -1.0, 0.5, 2.0], np.float32)
    vu = np.array([1.0, 1.0, 0.5, -2.0], np.float32)
    # v_u + w (v_c - v_u) at w = 2: 1 + 4, 1 - 4, 0.5 + 0, -2 + 8
    assert np.array_equal(O.cfg_combine(vc, vu, 2.0), np.array([5.0, -3.0, 0.5, 6.0], np.float32))
    r = np.random.default_rng(40)
    a, b = r.standard_normal(500).astype(np.float32), r.standard_normal(500).astype(np.float32)
    assert np.array_equal(O.cfg_combine(a, b, 0.0), b)  # w = 0: the unconditional branch exactly
    assert O.cfg_combine(a, b, 3.0).dtype == np.float32
    # float32 steps: each of the three operations rounds once
    d = (a - b).astype(np.float32)
    exact = b.astype(np.float64) + 3.0 * (a.astype(np.float64) - b.astype(np.float64))
    got = O.cfg_combine(a, b, 3.0).astype(np.float64)
    assert np.abs(got - exact).max() <= 4 * np.finfo(np.float32).eps * (np.abs(exact) + 3 * np.abs(d)).max()


def test_cfg_pairs_layout():
    c2 = S.get_config("c2")
    assert O.cfg_pairs(c2) == 1
    four = scaled(c2, segments=(Segment(0, (8,), 0), Segment(0, (12,), 0), Segment(0, (8,), 1),
                                Segment(0, (12,), 1)))
    assert O.cfg_pairs(four) == 2
    with pytest.raises(ValueError):
        O.cfg_pairs(scaled(c2, segments=four.segments[:3]))
    with pytest.raises(ValueError):  # segment j pairs with j + P, not j + 1
        O.cfg_pairs(scaled(c2, segments=(Segment(0, (8,), 0), Segment(0, (8,), 1), Segment(0, (12,), 0),
                                         Segment(0, (12,), 1))))


_CFG_TINY = scaled(S.get_config("c2"), n_blocks=1, hidden=256, n_heads=2, ffn=512, denoise_steps=3,
                   segments=(Segment(0, (8,), 0), Segment(0, (12,), 0), Segment(0, (8,), 1),
                             Segment(0, (12,), 1)))


def _cfg_setup(cfg):
    isl = S.island_weights(cfg)
    bw = S.block_weights(cfg, 0)
    inp = S.inputs(cfg)
    P = len(cfg.segments) // 2
    lat = {f"latent.{j}": inp[f"latent.{j}"] for j in range(P)}
    conds = S.cond_steps(cfg, cfg.denoise_steps)
    dt = O.sigma_dt(O.sigma_schedule(cfg.shifts[0], cfg.denoise_steps))
    dts = dt[:, None]
    return isl, (lambda b: bw), lat, conds, dts


def _alone_loop(cfg, j, source, W, isl, lat, conds, dts, n):
    """Segment j on its own with conditioning source ``source``: a plain Euler
    loop on the unguided velocity."""
    seg = cfg.segments[j]
    one = scaled(cfg, segments=(Segment(seg.modality, seg.grid, 0),), cond_rows=(CondRow(seg.modality, 0),),
                 cfg_replicate_latent=False)
    x = lat[f"latent.{j}"]
    for i in range(n):
        v = O.forward(one, W, isl, {"latent.0": x, "cond": conds[i][source:source + 1]})["latent.0"]
        x = O.euler_step(x, v.astype(np.float32), dts[i][seg.modality])
    return x


def test_cfg_loop_reduces_to_each_branch():
    cfg = _CFG_TINY
    isl, W, lat, conds, dts = _cfg_setup(cfg)
    n = cfg.denoise_steps
    g0 = O.cfg_denoise_loop(cfg, W, isl, lat, conds, dts, 0.0, n)
    g1 = O.cfg_denoise_loop(cfg, W, isl, lat, conds, dts, 1.0, n)
    for j in range(2):
        unc = _alone_loop(cfg, j, 1, W, isl, lat, conds, dts, n)
        con = _alone_loop(cfg, j, 0, W, isl, lat, conds, dts, n)
        assert np.abs(con - unc).max() > 1e-3  # the two branches do differ
        # w = 0: the unconditional branch, up to the packed-vs-alone fp64 rounding order
        assert np.abs(g0[f"latent.{j}"] - unc).max() < 1e-6
        # w = 1: the conditional branch, up to three float32 roundings per step
        assert np.abs(g1[f"latent.{j}"] - con).max() < 1e-5


def test_cfg_loop_identical_branches_ignore_guidance():
    cfg = _CFG_TINY
    isl, W, lat, conds, dts = _cfg_setup(cfg)
    conds = conds.copy()
    conds[:, 1] = conds[:, 0]
    g = O.cfg_denoise_loop(cfg, W, isl, lat, conds, dts, 7.5, 2)
    for j in range(2):
        plain = _alone_loop(cfg, j, 0, W, isl, lat, conds, dts, 2)
        assert np.abs(g[f"latent.{j}"] - plain).max() < 1e-5


def test_cfg_step_is_affine_in_guidance():
    cfg = _CFG_TINY
    isl, W, lat, conds, dts = _cfg_setup(cfg)
    x = [O.cfg_denoise_loop(cfg, W, isl, lat, conds, dts, w, 1)["latent.1"].astype(np.float64) for w in (0.0, 1.0, 2.0)]
    step = x[1] - x[0]
    assert np.abs(step).max() > 1e-4
    assert np.abs((x[2] - x[1]) - step).max() < 1e-5 * np.abs(x[0]).max()
