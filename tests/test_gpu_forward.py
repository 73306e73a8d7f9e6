"""Whole-path parity through the C ABI (dit_forward / dit_block_forward /
dit_denoise_step / dit_denoise_loop) against the CPU oracle, plus the
bit-exact invariants: packed == alone, zero gate == identity, determinism,
Euler update bit-exact, device loop == separate steps.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from gpu_util import assert_bf16_parity, assert_bf16_parity_stats, assert_f32_close, rms
from synthetic.configs import CondRow, Segment, scaled

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def H():
    import harness
    from video_audio_gen_amd import dit
    dit.load()
    return harness


def _oracle(cfg, weights, inp, t_rows=None, accum="fp64"):
    isl = {k: v for k, v in weights.items() if not k.startswith("blocks.")}
    return O.forward(cfg, lambda b: weights, isl, inp, t_rows=t_rows, threads=8, accum=accum)


def _run(H, cfg, seed=0):
    w = S.all_weights(cfg, seed, threads=8)
    r = H.Runner(cfg, seed, model=_stage(H, cfg, w))
    r.forward()
    return r, w, r.output_numpy()


def _stage(H, cfg, w):
    from video_audio_gen_amd import dit
    m = dit.Model(cfg)
    dit.dit_stage_weights(m, w, as_bf16=cfg.stream == "bf16")
    dit.dit_stage_finalize(m)
    return m


C3_SMALL = scaled(S.get_config("c3"), segments=(Segment(0, (2, 8, 16), 0), Segment(1, (64,), 1)))
C4_SMALL = scaled(S.get_config("c4"), n_blocks=2,
                  segments=(Segment(0, (1, 4, 8), 0), Segment(1, (24,), 1), Segment(0, (2, 2, 4), 2),
                            Segment(1, (40,), 3)))
C5_SMALL = scaled(S.get_config("c5"), n_blocks=2, hidden=256, n_heads=2, ffn=512, denoise_steps=4,
                  segments=(Segment(0, (2, 4, 8), 0), Segment(1, (16,), 1)))


def test_c1_tiny_f32_parity(H):
    cfg = S.get_config("c1")
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    assert_f32_close(got["x"], ref["x"], what="c1 forward")
    c = H.dit.dit_counters()
    assert c["gemm_f32"] > 0 and c["attention_f32"] > 0
    # the fp32 stream's fused row kernels ran: residual + norm + slices, SiLU + slices
    assert c["resid_norm_slice"] > 0 and c["silu_slice"] > 0


# fp32 stream at widths that reach the fused row kernels' rarer paths: an ffn
# that is not a multiple of 32 (zero slices pad the MLP-out GEMM's K), more
# than eight split-K partials (MLP out: 96 x 8200 takes 32 splits), LayerNorm
# and the swapped [value | gate] projection.
C1_RAGGED = scaled(S.get_config("c1"), hidden=96, n_heads=3, ffn=8200, norm="layer", mlp="value_gate",
                   segments=(Segment(0, (3, 3, 4), 0), Segment(0, (2, 5, 5), 0)))


def test_f32_ragged_ffn_many_splits_parity(H):
    cfg = C1_RAGGED
    assert H.dit.dit_gemm_splits(cfg.hidden, cfg.ffn) > 8
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    assert_f32_close(got["x"], ref["x"], what="ragged fp32 forward")


def test_c2_music_f32_reduced_depth_parity(H):
    cfg = scaled(S.get_config("c2"), n_blocks=2)
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    for k in ref:
        assert_f32_close(got[k], ref[k], what=f"c2 (2 blocks) {k}")
    assert np.abs(got["latent.0"] - got["latent.1"]).max() > 1e-3  # CFG branches differ


def test_c2_music_f32_full_parity(H):
    cfg = S.get_config("c2")
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    for k in ref:
        err = np.abs(got[k] - ref[k])
        ratio = err / (1e-6 + 1e-5 * np.abs(ref[k]))
        print(f"c2 {k}: max|d| {err.max():.3e} rms {rms(ref[k]):.3e} worst err/bound {ratio.max():.3f} "
              f"outside {(ratio > 1).sum()}/{err.size}")
        assert_f32_close(got[k], ref[k], what=f"c2 full {k}")


def test_c3_block_bf16_parity(H):
    cfg = C3_SMALL
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    ctl = _oracle(cfg, w, r.inp, accum="fp32")
    assert_bf16_parity(got["x"], ref["x"], ctl["x"], "c3 block (320 tokens)")


def test_c4_io_bf16_parity(H):
    cfg = C4_SMALL
    r, w, got = _run(H, cfg)
    ref = _oracle(cfg, w, r.inp)
    ctl = _oracle(cfg, w, r.inp, accum="fp32")
    for k in ref:
        assert_bf16_parity(got[k], ref[k], ctl[k], f"c4 small (2 blocks) {k}")


def test_nonfinite_input_stays_visible_and_inside_its_document(H):
    """A NaN in one token of the fp32 tiny model's first document: every
    output of that document is NaN (attention mixes the document's rows, and
    the int8-sliced GEMMs carry a non-finite row as NaN rather than as finite
    digits), while the second document's outputs equal the clean forward's
    bit for bit (no term crosses a document boundary)."""
    cfg = S.get_config("c1")
    r, w, clean = _run(H, cfg)
    x = r.x_in.clone()
    x[5, 3] = float("nan")
    out = torch.empty_like(x)
    r.forward(x_in=x, out=out)
    got = r.output_numpy(out)["x"]
    n0 = cfg.segments[0].n_tokens
    assert np.isnan(got[:n0]).all()
    assert np.array_equal(got[n0:], clean["x"][n0:])


def test_packed_equals_alone_bits(H):
    for cfg in (S.get_config("c1"), C3_SMALL):
        w = S.all_weights(cfg, 0, threads=8)
        m = _stage(H, cfg, w)
        r = H.Runner(cfg, 0, model=m)
        r.forward()
        packed = r.output_numpy()["x"]
        lay = O.pack_layout(cfg)
        for i, seg in enumerate(cfg.segments):
            a, b = int(lay["cu_seqlens"][i]), int(lay["cu_seqlens"][i + 1])
            one = scaled(cfg, segments=(seg,))
            batch = H.dit.Batch(m, one.segments, H.cond_modality(cfg))
            ws = H.dit.workspace(batch)
            xi = r.x_in[a:b].contiguous()
            out = torch.empty_like(xi)
            H.dit.dit_forward(m, batch, xi, r.cond, out, ws)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), packed[a:b]), f"{cfg.name} segment {i}"


def test_zero_gate_block_identity_and_determinism(H):
    cfg = C3_SMALL
    w = S.all_weights(cfg, 0, threads=8)
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    mod = torch.randn(cfg.n_cond, 6, cfg.hidden, device="cuda")
    mod[:, 2] = 0
    mod[:, 5] = 0
    x = r.x_in.clone()
    H.dit.dit_block_forward(m, 0, x, mod, r.batch, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(x, r.x_in)
    a = r.forward().clone()
    b = r.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _schedule_tables(H, cfg):
    """Per-step conditioning rows and dt, built once on the host by the library."""
    dit = H.dit
    steps = cfg.denoise_steps
    sig = {m: dit.dit_sigma_schedule(cfg.shifts[m], steps) for m in range(cfg.n_mod)}
    conds, dts = [], []
    for i in range(steps):
        t_rows = [np.float32(sig[r.modality][0][i]) for r in cfg.cond_rows]
        conds.append(dit.dit_timestep_embedding(np.asarray(t_rows, np.float32), cfg.cond_dim))
        dts.append([sig[m][1][i] for m in range(cfg.n_mod)])
    return (torch.from_numpy(np.stack(conds)).cuda(), torch.from_numpy(np.asarray(dts, np.float32)).cuda())


def test_euler_steps_bit_exact_with_constant_velocity(H):
    # No blocks and a zero output projection make the velocity exactly the output
    # bias, on the GPU and in the oracle, so every Euler update must match bit for bit.
    cfg = scaled(C5_SMALL, n_blocks=0)
    w = S.island_weights(cfg)
    for mm in range(cfg.n_mod):
        w[f"out.{mm}.weight"][:] = 0.0
        w[f"out.{mm}.bias"][:] = np.random.default_rng(30 + mm).standard_normal(w[f"out.{mm}.bias"].shape)
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    cond_tab, dt_tab = _schedule_tables(H, cfg)
    lat = r.x_in.clone()
    for i in range(cfg.denoise_steps):
        H.dit.dit_denoise_step(m, r.batch, lat, cond_tab[i], dt_tab[i], r.ws)
        want = O.denoise_loop(cfg, lambda b: {}, w, r.inp, i + 1)
        got = H.unpack_output(cfg, lat.cpu().numpy())
        for k in want:
            assert np.array_equal(got[k], want[k]), f"step {i} {k}"


def test_denoise_loop_matches_steps_and_oracle(H):
    cfg = C5_SMALL
    w = S.all_weights(cfg, 0, threads=8)
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    cond_tab, dt_tab = _schedule_tables(H, cfg)
    lat = r.x_in.clone()
    for i in range(cfg.denoise_steps):
        H.dit.dit_denoise_step(m, r.batch, lat, cond_tab[i], dt_tab[i], r.ws)
    lat_loop = r.x_in.clone()
    H.dit.dit_denoise_loop(m, r.batch, lat_loop, cond_tab, dt_tab, cfg.denoise_steps, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(lat_loop, lat)  # the device loop is the same computation as single steps
    assert (lat - r.x_in).abs().max().item() > 1e-2  # the loop moves the latents
    isl = {k: v for k, v in w.items() if not k.startswith("blocks.")}
    ref = O.denoise_loop(cfg, lambda b: w, isl, r.inp, cfg.denoise_steps, threads=8)
    ctl = O.denoise_loop(cfg, lambda b: w, isl, r.inp, cfg.denoise_steps, threads=8, accum="fp32")
    got = H.unpack_output(cfg, lat.cpu().numpy())
    for k in ref:
        # compare the distance travelled (latent - noise), the part the model computed
        x0 = r.inp[k].astype(np.float64)
        assert_bf16_parity(got[k] - x0, ref[k] - x0, ctl[k] - x0, f"denoise {cfg.denoise_steps} steps {k}")


@pytest.mark.parametrize("name", ["c1", "c2_2blocks"])
def test_graph_replay_matches_eager(H, name):
    """One forward captured as a HIP graph and replayed three times, with eager
    forwards and synchronisations between the replays: every replay equals the
    eager output bit for bit (the forward launches no memset or allocation)."""
    cfg = S.get_config("c1") if name == "c1" else scaled(S.get_config("c2"), n_blocks=2)
    r, w, _ = _run(H, cfg)
    eager = r.forward().clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        r.forward()
    for _ in range(3):
        r.out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.out, eager)
        again = r.forward().clone()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(again, eager)


def _golden(name):
    """A stored oracle output (tests/golden/make_samples.py runs only the CPU
    oracle and its fp32-accumulation control arm; nothing comes from the GPU)."""
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(__file__), "golden")
    if here not in sys.path:
        sys.path.insert(0, here)
    import make_samples
    meta = json.load(open(os.path.join(here, f"{name}.json")))
    arrays = np.load(os.path.join(here, f"{name}.npz"))
    cfg = make_samples.GOLDENS[name]["cfg"]
    assert meta["config"] == cfg.name and meta["n_tokens"] == cfg.n_tokens and meta["n_blocks"] == cfg.n_blocks
    return cfg, meta, arrays


def _check_golden(got, meta, arrays, what):
    for k, t in meta["tensors"].items():
        assert_bf16_parity_stats(got[k], arrays[k], t["control_max_rel"], t["control_rms_rel"], f"{what} {k}")


def test_c3_full_size_rows_parity(H):
    """The single 6144-wide bf16 block at its full size (24,576 video + 2,048
    audio tokens): complete output rows at both ends of each document, on
    either side of the 256-query attention tiles and the 256-row GEMM tiles,
    and at seeded interior rows, against the stored oracle rows."""
    cfg, meta, arrays = _golden("c3_block_bf16_rows")
    r, w, got = _run(H, cfg)
    rows = meta["rows"]
    _check_golden({"x": got["x"][rows]}, meta, arrays, "c3 full size (rows)")


@pytest.fixture(scope="module")
def model64(H):
    """The 64-block bf16 DiT's weights, staged once for every test that runs it
    (the benchmark's batch, the denoise configuration, the full-depth golden)."""
    m = H.stage_model(S.get_config("c4"), 0, threads=16)
    yield m
    del m
    torch.cuda.empty_cache()


def test_c4_full_depth_parity(H, model64):
    """The 64-block model at its full width and depth on four small documents
    of both modalities (with the in/out projections), against the oracle's
    whole output latents."""
    cfg, meta, arrays = _golden("c4_full_depth_small_tokens")
    r = H.Runner(cfg, 0, model=model64)
    r.forward()
    _check_golden(r.output_numpy(), meta, arrays, "c4 64 blocks, 112 tokens")
    del r


@pytest.mark.parametrize("name", ["c4_full_tokens_2blocks", "c5_full_tokens_2blocks_step0"])
def test_full_token_layouts_parity(H, name):
    """The benchmark's packed layouts at 18,432 tokens -- two requests of
    8,192 video + 1,024 audio tokens in four documents, and one request of
    16,384 + 2,048 at the first denoise step (timesteps sigma(0)) -- through
    the first two blocks of the 64-block model's weights, whole output
    latents against the oracle's."""
    cfg, meta, arrays = _golden(name)
    w = {}
    m = H.stage_model(cfg, 0, threads=16)
    r = H.Runner(cfg, 0, model=m)
    cond = r.cond
    if meta["t_rows"] is not None:
        cond = torch.from_numpy(H.cond_rows(cfg, r.inp, meta["t_rows"])).cuda()
    r.forward(cond=cond)
    _check_golden(r.output_numpy(), meta, arrays, f"{name}")
    del r, m, w
    torch.cuda.empty_cache()


def test_c4_full_size_packed_equals_alone_and_deterministic(H, model64):
    """The 64-block bf16 DiT at its benchmark size (18,432 tokens in four
    documents): properties that hold at any size.  Each document's velocities
    from the packed forward equal, bit for bit, a forward of that document
    alone (every GEMM row, attention document and modulation row is
    independent of the rest of the batch); a repeated forward is
    bit-identical; every output is finite."""
    import synthetic.gen as G
    cfg = S.get_config("c4")
    m = model64
    r = H.Runner(cfg, 0, model=m)
    r.forward()
    torch.cuda.synchronize()
    packed = r.out.clone()
    assert torch.isfinite(packed).all()
    r.forward()
    torch.cuda.synchronize()
    assert torch.equal(r.out, packed), "repeated forward differs"
    sizes = [int(np.prod(G.segment_latent_shape(cfg, i))) for i in range(len(cfg.segments))]
    offs = np.concatenate([[0], np.cumsum(sizes)])
    for i in (1, 2):  # one audio and one video document, of different requests
        one = scaled(cfg, segments=(cfg.segments[i],))
        batch = H.dit.Batch(m, one.segments, H.cond_modality(cfg))
        ws = H.dit.workspace(batch)
        xi = r.x_in[offs[i]:offs[i + 1]].contiguous()
        out = torch.empty_like(xi)
        H.dit.dit_forward(m, batch, xi, r.cond, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, packed[offs[i]:offs[i + 1]]), f"document {i} alone differs from the packed forward"
        del ws


def test_c5_full_size_denoise_loop_equals_steps(H, model64):
    """The 50-step denoise configuration at its full size (64 blocks, 18,432
    tokens): the device loop over the first three steps equals three single
    steps bit for bit, the latents stay finite and move."""
    cfg = S.get_config("c5")
    m = model64
    r = H.Runner(cfg, 0, model=m)
    cond_tab, dt_tab = _schedule_tables(H, cfg)
    n = 3
    lat = r.x_in.clone()
    for i in range(n):
        H.dit.dit_denoise_step(m, r.batch, lat, cond_tab[i], dt_tab[i], r.ws)
    lat_loop = r.x_in.clone()
    H.dit.dit_denoise_loop(m, r.batch, lat_loop, cond_tab, dt_tab, n, r.ws)
    torch.cuda.synchronize()
    assert torch.isfinite(lat).all()
    assert torch.equal(lat_loop, lat)
    assert (lat - r.x_in).abs().max().item() > 1e-3


# ----------------------------------------------------------------------------- guided (CFG) loop

CFG_SMALL = scaled(S.get_config("c2"), n_blocks=2, hidden=256, n_heads=2, ffn=512, denoise_steps=30,
                   segments=(Segment(0, (86,), 0), Segment(0, (40,), 0), Segment(0, (86,), 1),
                             Segment(0, (40,), 1)))


def _cfg_tables(H, cfg, n):
    conds = S.cond_steps(cfg, n)
    cond_tab = torch.from_numpy(H.cond_step_rows(cfg, conds)).cuda()
    dts = H.dt_table(cfg, n)
    return conds, cond_tab, dts, torch.from_numpy(dts).cuda()


def _cfg_oracle_steps(cfg, w_model, lat, conds, dts, w, n):
    """The oracle's guided loop, step by step, keeping each step's two branch
    velocities for the error bound; checked equal to oracle.cfg_denoise_loop."""
    P = len(cfg.segments) // 2
    isl = {k: v for k, v in w_model.items() if not k.startswith("blocks.")}
    x = {k: np.asarray(v, np.float32) for k, v in lat.items()}
    vels = []
    for i in range(n):
        inp = {f"latent.{j}": x[f"latent.{j % P}"] for j in range(2 * P)}
        inp["cond"] = conds[i]
        v = O.forward(cfg, lambda b: w_model, isl, inp, threads=8)
        vels.append(v)
        for j in range(P):
            g = O.cfg_combine(v[f"latent.{j}"].astype(np.float32), v[f"latent.{j + P}"].astype(np.float32), w)
            x[f"latent.{j}"] = O.euler_step(x[f"latent.{j}"], g, np.float32(dts[i][0]))
    ref = O.cfg_denoise_loop(cfg, lambda b: w_model, isl, lat, conds, dts, w, n, threads=8)
    for k in ref:
        assert np.array_equal(ref[k], x[k])
    return x, vels


def _cfg_bound(cfg, vels, dts, w, x_ref):
    """Per element: each forward is inside |d| <= 1e-6 + 1e-5 |v|; the guided
    velocity (1 - w) v_u + w v_c carries |1 - w| and |w| of those; each step
    moves the latent by |dt| of that.  Doubled for the latent fed back into the
    later steps, plus one float32 rounding of the latent per step."""
    P = len(cfg.segments) // 2
    tol = {f"latent.{j}": np.zeros_like(x_ref[f"latent.{j}"], np.float64) for j in range(P)}
    for i, v in enumerate(vels):
        for j in range(P):
            vc = np.abs(v[f"latent.{j}"].astype(np.float64))
            vu = np.abs(v[f"latent.{j + P}"].astype(np.float64))
            tol[f"latent.{j}"] += abs(float(dts[i][0])) * (abs(1 - w) * (1e-6 + 1e-5 * vu) + abs(w) * (1e-6 + 1e-5 * vc))
    return {k: 2 * t + len(vels) * 2.0 ** -23 * np.abs(x_ref[k]) for k, t in tol.items()}


def test_cfg_loop_is_forward_then_guided_euler_bits(H):
    """One guided step equals dit_forward on the latents copied into both
    branches followed by the guidance combine and the Euler update done on
    the host in float32 (bit for bit); n steps of the loop equal n one-step
    calls; w = 1 equals the plain Euler step on the conditional velocity."""
    cfg = CFG_SMALL
    w_model = S.all_weights(cfg, 0, threads=8)
    m = _stage(H, cfg, w_model)
    r = H.Runner(cfg, 0, model=m)
    n = 3
    conds, cond_tab, dts, dt_tab = _cfg_tables(H, cfg, n)
    P = 2
    half = sum(int(np.prod(r.inp[f"latent.{j}"].shape)) for j in range(P))
    assert torch.equal(r.x_in[:half], r.x_in[half:])  # the batch's two halves hold one latent
    w = 3.5
    lat = r.x_in[:half].clone()
    H.dit.dit_cfg_denoise_loop(m, r.batch, lat, cond_tab[0], dt_tab[0], w, 1, r.ws)
    # the same step composed from the forward and host float32 arithmetic
    v = r.forward(x_in=r.x_in, cond=cond_tab[0]).cpu().numpy()
    vc, vu = v[:half], v[half:]
    d = (vc - vu).astype(np.float32)
    g = (vu + (np.float32(w) * d).astype(np.float32)).astype(np.float32)
    x0 = r.x_in[:half].cpu().numpy()
    want = (x0 + (np.float32(dts[0][0]) * g).astype(np.float32)).astype(np.float32)
    got = lat.cpu().numpy()
    assert np.array_equal(got, want)
    assert np.abs(got - x0).max() > 1e-3
    # n steps in one call == n one-step calls
    lat_loop = r.x_in[:half].clone()
    H.dit.dit_cfg_denoise_loop(m, r.batch, lat_loop, cond_tab, dt_tab, w, n, r.ws)
    lat_steps = r.x_in[:half].clone()
    for i in range(n):
        H.dit.dit_cfg_denoise_loop(m, r.batch, lat_steps, cond_tab[i], dt_tab[i], w, 1, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(lat_loop, lat_steps)
    # w = 1: the guided velocity is vu + fl(vc - vu), the conditional velocity
    # up to that one rounding
    lat1 = r.x_in[:half].clone()
    H.dit.dit_cfg_denoise_loop(m, r.batch, lat1, cond_tab[0], dt_tab[0], 1.0, 1, r.ws)
    g1 = (vu + (vc - vu).astype(np.float32)).astype(np.float32)
    want1 = (x0 + (np.float32(dts[0][0]) * g1).astype(np.float32)).astype(np.float32)
    assert np.array_equal(lat1.cpu().numpy(), want1)


def test_cfg_loop_rejects_unpaired_batch(H):
    cfg = scaled(CFG_SMALL, segments=(Segment(0, (86,), 0), Segment(0, (40,), 0), Segment(0, (40,), 1),
                                      Segment(0, (86,), 1)))
    w_model = S.all_weights(cfg, 0, threads=8)
    r = H.Runner(cfg, 0, model=_stage(H, cfg, w_model))
    _, cond_tab, _, dt_tab = _cfg_tables(H, cfg, 1)
    lat = r.x_in[:(86 + 40) * 128].clone()
    with pytest.raises(H.dit.DitError, match="do not pair"):
        H.dit.dit_cfg_denoise_loop(r.model, r.batch, lat, cond_tab, dt_tab, 2.0, 1, r.ws)
    with pytest.raises(H.dit.DitError, match="not finite"):
        H.dit.dit_cfg_denoise_loop(r.model, r.batch, lat, cond_tab, dt_tab, float("nan"), 1, r.ws)


@pytest.mark.parametrize("name", ["small_4seg", "c2_2blocks"])
def test_cfg_loop_oracle_parity(H, name):
    """Guided loop against the oracle's: the distance each latent travels
    inside the fp32 bound of every forward, carried through the guidance."""
    if name == "small_4seg":
        cfg, n, w = CFG_SMALL, 3, 3.5
    else:
        cfg, n, w = scaled(S.get_config("c2"), n_blocks=2), 2, 5.0
    w_model = S.all_weights(cfg, 0, threads=8)
    r = H.Runner(cfg, 0, model=_stage(H, cfg, w_model))
    conds, cond_tab, dts, dt_tab = _cfg_tables(H, cfg, n)
    P = len(cfg.segments) // 2
    lat_in = {f"latent.{j}": r.inp[f"latent.{j}"] for j in range(P)}
    half = sum(int(np.prod(v.shape)) for v in lat_in.values())
    lat = r.x_in[:half].clone()
    H.dit.dit_cfg_denoise_loop(r.model, r.batch, lat, cond_tab, dt_tab, w, n, r.ws)
    torch.cuda.synchronize()
    got = H.unpack_output(cfg, np.concatenate([lat.cpu().numpy(), lat.cpu().numpy()]))
    x_ref, vels = _cfg_oracle_steps(cfg, w_model, lat_in, conds, dts, w, n)
    tol = _cfg_bound(cfg, vels, dts, w, x_ref)
    for k in x_ref:
        x0 = lat_in[k].astype(np.float64)
        dg = got[k].astype(np.float64) - x0
        dr = x_ref[k].astype(np.float64) - x0
        assert np.abs(dr).max() > 1e-3
        ratio = np.abs(dg - dr) / tol[k]
        print(f"cfg {name} {k}: max|d| {np.abs(dg - dr).max():.3e} worst err/bound {ratio.max():.3f}")
        assert (ratio <= 1).all(), f"{k}: {(ratio > 1).sum()} outside the bound, worst {ratio.max():.3f}"


# ----------------------------------------------------------------------------- fused epilogues

def _with_biases(w, seed=7, scale=0.1):
    """The weights with every bias (block GEMMs, AdaLN, projections) drawn
    N(0, scale^2) instead of zero, so the bias paths carry values."""
    rng = np.random.default_rng(seed)
    out = dict(w)
    for k, v in w.items():
        if k.endswith(".bias"):
            out[k] = (rng.standard_normal(v.shape) * scale).astype(np.float32)
    return out


@pytest.mark.parametrize("name", ["c1_ragged_value_gate", "c3_small", "c4_small_io"])
def test_nonzero_biases_parity(H, name):
    """Every bias non-zero: oracle parity (fp32 bound, or the bf16 bound with
    its control arm), and the output moves against the zero-bias forward, so
    no bias path is dead -- including the MLP-in bias staged half-swapped
    ([value | gate] models) or in [32 gate | 32 up] groups (bf16 models)."""
    cfg = {"c1_ragged_value_gate": C1_RAGGED, "c3_small": C3_SMALL, "c4_small_io": C4_SMALL}[name]
    w0 = S.all_weights(cfg, 0, threads=8)
    w = _with_biases(w0)
    r = H.Runner(cfg, 0, model=_stage(H, cfg, w))
    r.forward()
    got = r.output_numpy()
    r0 = H.Runner(cfg, 0, model=_stage(H, cfg, w0))
    r0.forward()
    got0 = r0.output_numpy()
    ref = _oracle(cfg, w, r.inp)
    for k in ref:
        assert np.abs(got[k] - got0[k]).max() > 1e-3
        if cfg.stream == "f32":
            assert_f32_close(got[k], ref[k], what=f"{name} {k} with biases")
        else:
            ctl = _oracle(cfg, w, r.inp, accum="fp32")
            assert_bf16_parity(got[k], ref[k], ctl[k], f"{name} {k} with biases")


@pytest.mark.parametrize("name", ["c3_small", "ragged", "ragged_biases"])
def test_bf16_block_equals_separate_kernels_bits(H, name):
    """The bf16 block applies the SiLU gate inside the MLP-in GEMM's epilogue
    (its weight staged in [32 gate | 32 up] row groups); it equals the same
    block built from the op-level calls -- a GEMM that stores u on the plain
    [gate | up] weight, then the separate SiLU-gate kernel -- bit for bit,
    at a ragged width too (ffn 704: 5.5 column tiles of 256)."""
    cfg = C3_SMALL if name == "c3_small" else scaled(
        C3_SMALL, hidden=256, n_heads=2, ffn=704,
        segments=(Segment(0, (1, 5, 7), 0), Segment(1, (45,), 1), Segment(0, (2, 3, 9), 0)))
    w = S.all_weights(cfg, 0, threads=8)
    if name == "ragged_biases":
        w = _with_biases(w)
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    dit = H.dit
    N, D, F, nh, hd = cfg.n_tokens, cfg.hidden, cfg.ffn, cfg.n_heads, cfg.head_dim
    mod = torch.empty(1, r.batch.n_cond, 6, D, device="cuda")
    dit.dit_modulation(m, r.batch, 0, 1, r.cond, mod)
    x_blk = r.x_in.clone()
    dit.dit_block_forward(m, 0, x_blk, mod[0], r.batch, r.ws)

    lay = dit.dit_pack_layout(cfg)
    cos, sin = dit.dit_rope_cache_build(cfg)
    cu = torch.from_numpy(lay["cu_seqlens"]).cuda()
    ci = torch.from_numpy(lay["cond_idx"]).cuda()
    cos, sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    bw = lambda k: torch.from_numpy(w[f"blocks.0.{k}"]).cuda()
    wb = lambda k: bw(k).to(torch.bfloat16).contiguous()
    mod0 = mod[0].contiguous()
    norm = 0 if cfg.norm == "rms" else 1
    x = r.x_in.clone()
    h = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    dit.dit_modnorm(norm, cfg.norm_eps, x, mod0, 0, ci, h)
    qkv = torch.empty(N, 3 * D, dtype=torch.bfloat16, device="cuda")
    dit.dit_gemm(h, wb("attn.qkv.weight"), bw("attn.qkv.bias"), qkv)
    q, k, v = (torch.empty(nh, N, hd, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    dit.dit_rope_split(qkv, nh, hd, cfg.rot_dim, cos, sin, q, k, v)
    o = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(q, k, v, cu, r.batch.max_seqlen, o)
    a = torch.empty(N, D, dtype=torch.float32, device="cuda")
    dit.dit_gemm(o, wb("attn.out.weight"), bw("attn.out.bias"), a)
    dit.dit_gated_residual(x, a, mod0, 0, ci)
    dit.dit_modnorm(norm, cfg.norm_eps, x, mod0, 1, ci, h)
    u = torch.empty(N, 2 * F, dtype=torch.bfloat16, device="cuda")
    dit.dit_gemm(h, wb("mlp.in.weight"), bw("mlp.in.bias"), u)
    mm = torch.empty(N, F, dtype=torch.bfloat16, device="cuda")
    dit.dit_silu_gate(u, mm)
    dit.dit_gemm(mm, wb("mlp.out.weight"), bw("mlp.out.bias"), a)
    dit.dit_gated_residual(x, a, mod0, 1, ci)
    torch.cuda.synchronize()
    assert (x - r.x_in).abs().max().item() > 1e-3
    assert torch.equal(x_blk, x)


def test_cfg_loop_graph_replay_matches_eager(H):
    """Three guided steps captured as one HIP graph (two device copies, the
    forward's kernels and the guided Euler kernel per step) replay equal to
    the eager loop bit for bit, three times, with eager loops between."""
    cfg = CFG_SMALL
    w_model = S.all_weights(cfg, 0, threads=8)
    r = H.Runner(cfg, 0, model=_stage(H, cfg, w_model))
    n = 3
    _, cond_tab, _, dt_tab = _cfg_tables(H, cfg, n)
    half = r.x_in.numel() // 2
    lat = r.x_in[:half].clone()
    H.dit.dit_cfg_denoise_loop(r.model, r.batch, lat, cond_tab, dt_tab, 3.5, n, r.ws)
    torch.cuda.synchronize()
    eager = lat.clone()
    g_lat = r.x_in[:half].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        H.dit.dit_cfg_denoise_loop(r.model, r.batch, g_lat, cond_tab, dt_tab, 3.5, n, r.ws)
    for _ in range(3):
        g_lat.copy_(r.x_in[:half])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_lat, eager)
        again = r.x_in[:half].clone()
        H.dit.dit_cfg_denoise_loop(r.model, r.batch, again, cond_tab, dt_tab, 3.5, n, r.ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)


@pytest.mark.parametrize("name", ["c2_2blocks", "c4_small"])
def test_adaln_table_correctly_rounded(H, name):
    """dit_modulation against the oracle's table on the same float32
    conditioning rows: fp64 dot products rounded once, so at most one ulp
    apart (sums in another order) and almost every value identical; with
    random biases so the bias term is live."""
    cfg = scaled(S.get_config("c2"), n_blocks=2) if name == "c2_2blocks" else C4_SMALL
    w = _with_biases(S.all_weights(cfg, 0, threads=8))
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    L, D = cfg.n_blocks, cfg.hidden
    mod = torch.empty(L, r.batch.n_cond, 6, D, device="cuda")
    H.dit.dit_modulation(m, r.batch, 0, L, r.cond, mod)
    got = mod.cpu().numpy()
    emb = r.cond.cpu().numpy().astype(np.float64)
    same = total = 0
    for b in range(L):
        ref = O.adaln_table(cfg, w, b, emb, "fp64").astype(np.float32)
        ulp = np.spacing(np.abs(ref)).astype(np.float64)
        assert (np.abs(got[b].astype(np.float64) - ref) <= ulp).all(), f"block {b}: beyond one ulp"
        same += int((got[b] == ref).sum())
        total += ref.size
    assert same >= 0.999 * total, f"{total - same} of {total} values differ by one ulp"


def test_bf16_forward_equals_block_by_block_bits(H):
    """dit_forward of a bf16 model runs each MLP's gated residual fused with
    the next block's attention norm; it equals dit_block_forward called block
    after block (each closing with the separate gated residual) bit for bit."""
    cfg = scaled(C3_SMALL, n_blocks=3, hidden=256, n_heads=2, ffn=704)
    w = _with_biases(S.all_weights(cfg, 0, threads=8))
    m = _stage(H, cfg, w)
    r = H.Runner(cfg, 0, model=m)
    out = r.forward().clone()
    mod = torch.empty(cfg.n_blocks, r.batch.n_cond, 6, cfg.hidden, device="cuda")
    H.dit.dit_modulation(m, r.batch, 0, cfg.n_blocks, r.cond, mod)
    x = r.x_in.clone()
    for b in range(cfg.n_blocks):
        H.dit.dit_block_forward(m, b, x, mod[b].contiguous(), r.batch, r.ws)
    torch.cuda.synchronize()
    assert (out - r.x_in).abs().max().item() > 1e-3
    assert torch.equal(out, x)


@pytest.mark.parametrize("name", ["c1", "c4_small"])
def test_forward_graph_replays_match_eager(H, name):
    """dit_forward captured by the library as one HIP graph
    (dit_forward_graph_create) replays equal to the eager forward bit for bit,
    three times with eager forwards between; a replay after new latents are
    written into the captured input equals the eager forward of those
    latents."""
    dit = H.dit
    cfg = S.get_config("c1") if name == "c1" else C4_SMALL
    w = S.all_weights(cfg, 0, threads=8)
    r = H.Runner(cfg, 0, model=_stage(H, cfg, w))
    eager = r.forward().clone()
    torch.cuda.synchronize()
    out = torch.empty_like(r.out)
    g = dit.ForwardGraph(r.model, r.batch, r.x_in, r.cond, out, r.ws)
    assert g.nodes > 0
    for _ in range(3):
        out.fill_(float("nan"))
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        again = r.forward()  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        assert torch.equal(again, eager)
    x0 = r.x_in.clone()
    r.x_in.mul_(0.5)
    want = r.forward().clone()
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(out, want) and not torch.equal(want, eager)
    r.x_in.copy_(x0)
    g.close()


def test_forward_graph_refused_while_profiling(H):
    """Per-launch profiling records events at every launch, which a capture
    would swallow: creating a graph then fails with DIT_E_UNSUPPORTED and
    launches nothing."""
    dit = H.dit
    cfg = S.get_config("c1")
    r = H.Runner(cfg, 0, model=_stage(H, cfg, S.all_weights(cfg, 0, threads=8)))
    dit.dit_profile_begin()
    try:
        with pytest.raises(dit.DitError) as e:
            dit.ForwardGraph(r.model, r.batch, r.x_in, r.cond, r.out, r.ws)
        assert e.value.status == "DIT_E_UNSUPPORTED" and "profil" in str(e.value)
    finally:
        dit.dit_profile_end()
