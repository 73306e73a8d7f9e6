"""Pins of the oracle's wiring: which tensor each step reads and where a bf16
block stream rounds.

Each expected value here is computed by a route of its own, not by retyping
the oracle's code: attention scores through complex numbers and the relative
position (so the roles of q and k and the target of RoPE are fixed by the
mathematics of rotary embeddings, page "port the MiniMax-H3 omni-modal
video+audio DiT", section "The device-resident forward (W2b)": RoPE from a
per-row cos/sin cache on q and k), patchify and unpatchify by explicit index
loops, bf16 rounding by ``math.frexp`` (not the oracle's bit trick), sigmas by
hand fractions.  Every test names the mutations of the oracle it catches; each
was checked by running the test against an oracle carrying that mutation.
"""

import math

import numpy as np

import oracle as O
import synthetic as S
from synthetic.configs import CondRow, DitConfig, Modality, Segment, scaled


def _bf16(v: float) -> float:
    """Nearest bf16 value (8 significant bits, ties to even), by frexp."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)           # v = m 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)   # round() is ties-to-even


def _f32(v: float) -> float:
    return float(np.float32(v))


def _rms_rows(x, eps):
    return x / np.sqrt((x * x).sum(axis=1, keepdims=True) / x.shape[1] + eps)


def _silu(z):
    return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------- (a) q/k roles, RoPE target

def _attn_cfg(**kw):
    # D 8, two heads of 4, all four dims rotary (two frequencies 1 and 1/100);
    # two documents of different modalities at positions 0..2 and 0..1
    base = dict(name="wiring", key_id=98, model_id=98, n_blocks=1, hidden=8, n_heads=2, head_dim=4, ffn=8,
                norm="rms", norm_eps=1e-6, mlp="gate_up", rot_dim=4, theta=10000.0, stream="f32",
                cond_kind="timestep", cond_dim=4,
                modalities=(Modality("a", "none", 0, (1, 1, 1), (4,)), Modality("b", "none", 0, (1, 1, 1), (4,))),
                segments=(Segment(0, (3,), 0), Segment(1, (2,), 1)),
                cond_rows=(CondRow(0, 0), CondRow(1, 0)), n_requests=1, io=False)
    base.update(kw)
    return DitConfig(**base)


def _attn_weights(rng, D, F):
    W = {"attn.qkv.weight": rng.standard_normal((3 * D, D)) * 0.8, "attn.qkv.bias": rng.standard_normal(3 * D) * 0.1,
         "attn.out.weight": rng.standard_normal((D, D)) * 0.5, "attn.out.bias": rng.standard_normal(D) * 0.1,
         "mlp.in.weight": rng.standard_normal((2 * F, D)) * 0.5, "mlp.in.bias": rng.standard_normal(2 * F) * 0.1,
         "mlp.out.weight": rng.standard_normal((D, F)) * 0.5, "mlp.out.bias": rng.standard_normal(D) * 0.1}
    return {"blocks.0." + k: v for k, v in W.items()}


def _attention_by_relative_position(q, k, v, pos, docs, hd, rot, theta, swap=False, rope_v=False, rope_k=True):
    """o[n] = sum over keys m of n's document of softmax_m(s_nm) v[m], with the
    rotary score written through complex numbers: pairing dims j and j + rot/2
    as z_j = x_j + i x_{j+rot/2}, RoPE multiplies z_j by e^{i p f_j}, so
    s_nm = Re sum_j zq_j(n) conj(zk_j(m)) e^{i (p_n - p_m) f_j} / sqrt(hd)
    plus the pass-through dims (none here: rot = hd).  The flags build the
    mutated variants the test must tell apart."""
    half = rot // 2
    f = [theta ** (-(2.0 * j) / rot) for j in range(half)]
    N, H, _ = q.shape
    if swap:
        q, k = k, q  # q and k trade roles
    o = np.zeros_like(v)
    for (a, b) in docs:
        for h in range(H):
            for n in range(a, b):
                s = []
                for m in range(a, b):
                    acc = 0.0
                    for j in range(half):
                        zq = complex(q[n, h, j], q[n, h, j + half])
                        zk = complex(k[m, h, j], k[m, h, j + half])
                        dp = pos[n] - (pos[m] if rope_k else 0.0)
                        acc += (zq * zk.conjugate() * complex(math.cos(dp * f[j]), math.sin(dp * f[j]))).real
                    s.append(acc / math.sqrt(hd))
                mx = max(s)
                e = [math.exp(t - mx) for t in s]
                tot = sum(e)
                for i, m in enumerate(range(a, b)):
                    vm = v[m, h].copy()
                    if rope_v:
                        for j in range(half):
                            z = complex(vm[j], vm[j + half]) * complex(math.cos(pos[m] * f[j]), math.sin(pos[m] * f[j]))
                            vm[j], vm[j + half] = z.real, z.imag
                    o[n, h] += (e[i] / tot) * vm
    return o


def _block_by_hand(cfg, x, mod, W, pos, docs, **mut):
    D, H, hd, F = cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.ffn
    ci = O.pack_layout(cfg)["cond_idx"]
    mt = mod[ci]
    w = lambda n: W["blocks.0." + n]  # noqa: E731
    h = _rms_rows(x, cfg.norm_eps) * (1 + mt[:, 1]) + mt[:, 0]
    qkv = h @ w("attn.qkv.weight").T + w("attn.qkv.bias")
    q, k, v = (qkv[:, i * D:(i + 1) * D].reshape(-1, H, hd) for i in range(3))
    o = _attention_by_relative_position(q, k, v, pos, docs, hd, cfg.rot_dim, cfg.theta, **mut).reshape(-1, D)
    x1 = x + mt[:, 2] * (o @ w("attn.out.weight").T + w("attn.out.bias"))
    h2 = _rms_rows(x1, cfg.norm_eps) * (1 + mt[:, 4]) + mt[:, 3]
    u = h2 @ w("mlp.in.weight").T + w("mlp.in.bias")
    m = _silu(u[:, :F]) * u[:, F:]
    return x1 + mt[:, 5] * (m @ w("mlp.out.weight").T + w("mlp.out.bias"))


def test_block_attention_roles_and_rope_target_by_relative_position():
    """A whole block on a 3-token and a 2-token document at positions 0..2 and
    0..1, with random q/k/v/out/MLP weights, against a hand computation whose
    scores use RoPE only through the query-key position difference.

    Mutations of the oracle this catches (each checked, and each variant below
    shown to move the result by far more than the tolerance): q and k swapped
    (scores transposed), RoPE applied to v as well, RoPE skipped on k.  (A
    document's positions shifted as a whole change nothing here, by the
    relative-position property; the grid's origin is pinned on the cache.)"""
    cfg = _attn_cfg()
    rng = np.random.default_rng(101)
    D = cfg.hidden
    x = rng.standard_normal((5, D))
    mod = rng.standard_normal((2, 6, D)) * 0.4
    W = _attn_weights(rng, D, cfg.ffn)
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    pos = [0.0, 1.0, 2.0, 0.0, 1.0]
    docs = [(0, 3), (3, 5)]
    want = _block_by_hand(cfg, x, mod, W, pos, docs)
    # with an fp64 cos/sin table of the same angles the block agrees to rounding ...
    f = [cfg.theta ** (-(2.0 * j) / cfg.rot_dim) for j in range(cfg.rot_dim // 2)]
    c64 = np.array([[math.cos(p * fj) for fj in f] for p in pos])
    s64 = np.array([[math.sin(p * fj) for fj in f] for p in pos])
    got = O.block_forward(cfg, x, mod, W, 0, lay, c64, s64, "fp64")
    assert np.abs(got - want).max() < 1e-12 * np.abs(want).max()
    # ... and with the oracle's own float32 cache to the cache's rounding
    got = O.block_forward(cfg, x, mod, W, 0, lay, cos, sin, "fp64")
    assert np.abs(got - want).max() < 1e-6 * np.abs(want).max()
    # the pin discriminates: every mutation moves the block output visibly
    for mut in (dict(swap=True), dict(rope_v=True), dict(rope_k=False)):
        bad = _block_by_hand(cfg, x, mod, W, pos, docs, **mut)
        assert np.abs(bad - want).max() > 1e-4, mut


# ----------------------------------------------------------------------------- (b) islands and final norm

def _io_cfg(norm="rms", n_blocks=0):
    # D 16; video: C 2, patch (1,2,2) -> token width 8; audio: C 4, channel-major -> width 4
    return DitConfig(
        name="islands", key_id=97, model_id=97, n_blocks=n_blocks, hidden=16, n_heads=2, head_dim=8, ffn=16,
        norm=norm, norm_eps=1e-6, mlp="gate_up", rot_dim=8, theta=10000.0, stream="f32", cond_kind="timestep",
        cond_dim=8,
        modalities=(Modality("video", "patch3d", 2, (1, 2, 2), (2, 2, 4)),
                    Modality("audio", "channel_major", 4, (1, 1, 1), (8,))),
        segments=(Segment(0, (2, 2, 3), 0), Segment(1, (5,), 1), Segment(0, (1, 3, 2), 0)),
        cond_rows=(CondRow(0, 0), CondRow(1, 0)), n_requests=1, io=True)


def _island_weights():
    I8, I4, Z4 = np.eye(8), np.eye(4), np.zeros((4, 4))
    rng = np.random.default_rng(102)
    return {
        # video: x = [t, 2t]; read back the first half, plus a bias
        "in.0.weight": np.vstack([I8, 2 * I8]), "in.0.bias": np.zeros(16),
        "out.0.weight": np.hstack([I8, np.zeros((8, 8))]), "out.0.bias": rng.standard_normal(8) * 0.1,
        # audio: x = [t, 0, 0, 3t]; read back the last quarter
        "in.1.weight": np.vstack([I4, Z4, Z4, 3 * I4]), "in.1.bias": np.zeros(16),
        "out.1.weight": np.hstack([Z4, Z4, Z4, I4]), "out.1.bias": rng.standard_normal(4) * 0.1,
    }


def _patch_tokens_by_loops(lat, grid, patch):
    C = lat.shape[0]
    T, Hh, Ww = grid
    pt, ph, pw = patch
    tok = []
    for t in range(T):
        for h in range(Hh):
            for w in range(Ww):
                vec = []
                for a in range(pt):
                    for b in range(ph):
                        for c in range(pw):
                            for ch in range(C):
                                vec.append(lat[ch, t * pt + a, h * ph + b, w * pw + c])
                tok.append(vec)
    return np.array(tok)


def _unpatch_by_loops(tok, C, grid, patch):
    T, Hh, Ww = grid
    pt, ph, pw = patch
    out = np.zeros((C, T * pt, Hh * ph, Ww * pw))
    n = 0
    for t in range(T):
        for h in range(Hh):
            for w in range(Ww):
                i = 0
                for a in range(pt):
                    for b in range(ph):
                        for c in range(pw):
                            for ch in range(C):
                                out[ch, t * pt + a, h * ph + b, w * pw + c] = tok[n, i]
                                i += 1
                n += 1
    return out


def test_forward_islands_and_final_norm_closed_form():
    """With in-projections x = [t, 2t] (video) and [t, 0, 0, 3t] (audio) and
    out-projections that read t's slot back, the forward is, per token,
    v = t / sqrt(5|t|^2/16 + eps) + b (video) and 3t / sqrt(10|t|^2/16 + eps) + b
    (audio) under RMSNorm, and (t - mean-of-x terms) under LayerNorm as written
    below, routed through patchify, packing, gather and unpatchify.

    Mutations this catches: the final norm dropped (v = t + b), the norm taken
    of the out-projection's input tokens instead of the residual stream, the
    two modalities' projections exchanged, a segment scattered to or gathered
    from the wrong packed rows, a wrong patch vector order."""
    for norm in ("rms", "layer"):
        for n_blocks in (0, 1):
            cfg = _io_cfg(norm, n_blocks)
            isl = _island_weights()
            D = cfg.hidden
            bw = {f"blocks.0.{k}": np.zeros(s) for k, s in S.gen.block_weight_shapes(cfg)}
            rng = np.random.default_rng(103)
            # a zero-gate block is the identity: its AdaLN rows are non-zero except both gates
            for mm in range(cfg.n_mod):
                Wa = rng.standard_normal((6 * D, cfg.cond_dim))
                Wa[2 * D:3 * D] = 0
                Wa[5 * D:6 * D] = 0
                bw[f"blocks.0.adaln.{mm}.weight"] = Wa
            for k in ("attn.qkv.weight", "attn.out.weight", "mlp.in.weight", "mlp.out.weight"):
                bw["blocks.0." + k] = rng.standard_normal(bw["blocks.0." + k].shape)
            inp = {"t": np.array([0.3], np.float32)}
            for i, s in enumerate(cfg.segments):
                inp[f"latent.{i}"] = rng.standard_normal(S.gen.segment_latent_shape(cfg, i))
            got = O.forward(cfg, lambda b: bw, isl, inp)
            eps = cfg.norm_eps
            for i, s in enumerate(cfg.segments):
                lat = inp[f"latent.{i}"]
                if s.modality == 0:
                    t = _patch_tokens_by_loops(lat, s.grid, (1, 2, 2))
                    x = np.hstack([t, 2 * t])
                    sl, b = slice(0, 8), isl["out.0.bias"]
                else:
                    t = lat.T.copy()
                    x = np.hstack([t, 0 * t, 0 * t, 3 * t])
                    sl, b = slice(12, 16), isl["out.1.bias"]
                if norm == "rms":
                    y = x / np.sqrt((x * x).sum(axis=1, keepdims=True) / D + eps)
                else:
                    c = x - x.sum(axis=1, keepdims=True) / D
                    y = c / np.sqrt((c * c).sum(axis=1, keepdims=True) / D + eps)
                v = y[:, sl] + b
                want = _unpatch_by_loops(v, 2, s.grid, (1, 2, 2)) if s.modality == 0 else v.T
                assert np.abs(got[f"latent.{i}"] - want).max() < 1e-12, (norm, n_blocks, i)
                # discriminates a dropped final norm
                no_norm = x[:, sl] + b
                no_norm = _unpatch_by_loops(no_norm, 2, s.grid, (1, 2, 2)) if s.modality == 0 else no_norm.T
                assert np.abs(no_norm - want).max() > 0.1


# ----------------------------------------------------------------------------- (c) bf16 storage points

def _bf(a):
    return np.vectorize(_bf16)(np.asarray(a, np.float64))


def _fl32(a):
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def _bf16_block_by_hand(cfg, x, mod, W, pos, docs, skip=(), extra=()):
    """One block of a bf16 stream with every storage point written out:
    h, qkv, q and k after RoPE, o, h2, u and m rounded to bf16; the residual x
    rounded to fp32 after each gated add; a and a2 (the projections feeding
    the residual) kept exact.  ``skip`` drops named bf16 roundings and
    ``extra`` adds bf16 roundings of a, a2 or x, to show each point matters."""
    D, H, hd, F = cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.ffn
    ci = O.pack_layout(cfg)["cond_idx"]
    mt = mod[ci]
    w = lambda n: W["blocks.0." + n]  # noqa: E731
    R = lambda name, a: a if name in skip else _bf(a)  # noqa: E731
    E = lambda name, a: _bf(a) if name in extra else a  # noqa: E731
    h = R("h", _rms_rows(x, cfg.norm_eps) * (1 + mt[:, 1]) + mt[:, 0])
    qkv = R("qkv", h @ w("attn.qkv.weight").T + w("attn.qkv.bias"))
    q, k, v = (qkv[:, i * D:(i + 1) * D].reshape(-1, H, hd) for i in range(3))
    # RoPE by explicit rotation of each (j, j + rot/2) pair
    half = cfg.rot_dim // 2
    f = [cfg.theta ** (-(2.0 * j) / cfg.rot_dim) for j in range(half)]
    qr, kr = q.copy(), k.copy()
    for n in range(q.shape[0]):
        for j in range(half):
            c, s = _f32(math.cos(pos[n] * f[j])), _f32(math.sin(pos[n] * f[j]))
            for src, dst in ((q, qr), (k, kr)):
                a, b = src[n, :, j], src[n, :, j + half]
                dst[n, :, j] = a * c - b * s
                dst[n, :, j + half] = b * c + a * s
    qr, kr = R("q", qr), R("k", kr)
    o = np.zeros_like(v)
    for (a0, b0) in docs:
        for hh in range(H):
            sc = qr[a0:b0, hh] @ kr[a0:b0, hh].T / math.sqrt(hd)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            o[a0:b0, hh] = (p / p.sum(axis=1, keepdims=True)) @ v[a0:b0, hh]
    o = R("o", o.reshape(-1, D))
    a = E("a", o @ w("attn.out.weight").T + w("attn.out.bias"))
    x1 = _fl32(x + mt[:, 2] * a)
    x1 = E("x", x1)
    h2 = R("h2", _rms_rows(x1, cfg.norm_eps) * (1 + mt[:, 4]) + mt[:, 3])
    u = R("u", h2 @ w("mlp.in.weight").T + w("mlp.in.bias"))
    m = R("m", _silu(u[:, :F]) * u[:, F:])
    a2 = E("a2", m @ w("mlp.out.weight").T + w("mlp.out.bias"))
    return E("x", _fl32(x1 + mt[:, 5] * a2))


def test_bf16_storage_points_by_hand():
    """The oracle's 'bf16' mode against a block whose storage points are
    written out by hand (bf16 rounding by frexp).  Documents of 6 and 5 tokens
    at positions 0..5 and 0..4 and non-representable weights, so that every
    rounding changes values that survive the later ones.

    Mutations this catches (each variant below moves the output by more than
    100x the tolerance, and each was checked against a mutated oracle): any one
    of the bf16 roundings of h, qkv, q, k, o, h2, u or m removed; a, a2 or x
    rounded to bf16 instead of kept in fp32."""
    cfg = _attn_cfg(stream="bf16", segments=(Segment(0, (6,), 0), Segment(1, (5,), 1)))
    rng = np.random.default_rng(104)
    D = cfg.hidden
    x = _fl32(rng.standard_normal((11, D)))
    mod = _fl32(rng.standard_normal((2, 6, D)) * 0.4)
    W = {k: _bf(v) if k.endswith("weight") else _fl32(v) for k, v in _attn_weights(rng, D, cfg.ffn).items()}
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    got = O.block_forward(cfg, x, mod, W, 0, lay, cos, sin, "bf16")
    pos = [0.0, 1.0, 2.0, 3.0, 4.0, 5.0, 0.0, 1.0, 2.0, 3.0, 4.0]
    docs = [(0, 6), (6, 11)]
    want = _bf16_block_by_hand(cfg, x, mod, W, pos, docs)
    tol = 1e-9 * np.abs(want).max()
    assert np.abs(got - want).max() <= tol
    for name in ("h", "qkv", "q", "k", "o", "h2", "u", "m"):
        bad = _bf16_block_by_hand(cfg, x, mod, W, pos, docs, skip=(name,))
        assert np.abs(bad - want).max() > 100 * tol, name
    for name in ("a", "a2", "x"):
        bad = _bf16_block_by_hand(cfg, x, mod, W, pos, docs, extra=(name,))
        assert np.abs(bad - want).max() > 100 * tol, name


def test_bf16_rounding_helper_agrees_with_frexp_rounding():
    r = np.random.default_rng(105).standard_normal(5000) * 7
    assert np.array_equal(O.round_bf16(r), _bf(r))


# ----------------------------------------------------------------------------- (d) denoise step conditions

def test_denoise_step_conditions_hand_values():
    """At step i the rows carry sigma_m(i) (not sigma_m(i+1)) and the step
    moves by sigma_m(i+1) - sigma_m(i).  Hand fractions for 50 steps, step 10:
    s = 0.8 -> video (shift 12) 9.6/9.8, audio (shift 3) 2.4/2.6; step 11:
    s = 0.78 -> 9.36/9.58 and 2.34/2.56.

    Mutations this catches: the next step's sigma used as the timestep, the
    shifts of the two modalities exchanged, dt of the wrong sign or step."""
    cfg = S.get_config("c5")
    t_rows, dts = O.denoise_step_conditions(cfg, 10)
    assert t_rows == [_f32(9.6 / 9.8), _f32(2.4 / 2.6)]
    assert dts[0] == np.float32(9.36 / 9.58 - 9.6 / 9.8)
    assert dts[1] == np.float32(2.34 / 2.56 - 2.4 / 2.6)
    t0, _ = O.denoise_step_conditions(cfg, 0)
    assert t0 == [1.0, 1.0]
    t49, d49 = O.denoise_step_conditions(cfg, 49)
    # s = 1/50: video 12/50 / (1 + 11/50) = 12/61, audio 3/50 / (1 + 2/50) = 3/52; the last step lands on 0
    assert t49 == [_f32(12 / 61), _f32(3 / 52)]
    assert d49[0] == np.float32(-12 / 61) and d49[1] == np.float32(-3 / 52)
