"""Benchmark of the DiT forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

One step is one full DiT forward (every block, with the projections in and
out) over one batch of seeded synthetic input whose weights and inputs were
staged to HBM before timing.  The default workload is the music-style fp32
acoustic DiT (24 blocks, hidden 2560, 20 heads x 128, ffn 10240, LayerNorm,
partial rotary on 64 dims, 2 CFG branches x 86 frames = 172 tokens): the
configuration the pages time (page "the 2.4B fp32 DiT onto the device, staged
once", section "Speed").

Prints one JSON line.  `value` is tokens per second (tokens of the batch /
seconds per forward); `roofline` reports the kernel family that takes the most
device time, from per-launch HIP events recorded on the launch stream during a
second pass of K forwards; `cpu_baseline` times the CPU oracle: for an fp32
workload one whole forward on one host thread (as the pages time theirs), for
a bf16 one a bounded sample of blocks on all host threads, scaled to a forward.

`--extra c4,c4_mxfp8` (the default) then frees the headline model and times the
64-block bf16 DiT (18,432 tokens in four documents, weights staged once), and
the same model with its block GEMMs on MXFP8 operands, each in a timed region
of its own, reported under `extra.<name>` with its own roofline: further
measured configurations, not part of the headline value.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms per DiT forward + tokens/s at 1 GPU; % of MFMA / HBM peak"
# MI355X published peaks.
PEAK = {"mfma_f64": 78.6, "mfma_bf16": 2500.0, "mfma_f32": 157.3, "mfma_i8": 5000.0, "mfma_fp8": 5000.0,
        "hbm_gbs": 8000.0,
        # the fp32 GEMM runs each fp32 product as 15 exact int8 slice products:
        # its ceiling in fp32 flop/s is the int8 MFMA peak / 15
        "mfma_i8_slices": 5000.0 / 15}
GEMM_FAMILY_PEAK = {"gemm_f32": ("mfma_i8_slices", "int8 MFMA 5.0 POP/s / 15 slice products per fp32 product"),
                    "gemm_bf16": ("mfma_bf16", "bf16 MFMA"),
                    "gemm_mx8": ("mfma_fp8", "fp8 MFMA (MXFP8 operands)"),
                    "gemm_mx4": ("mfma_fp8", "fp8 MFMA (MXFP8 activations x MXFP4 weights run at the fp8 rate)"),
                    "attention_bf16": ("mfma_bf16", "bf16 MFMA")}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


KERNEL_SOURCE = {"gemm_f32": "video_audio_gen_amd/csrc/gemm_slices.hip", "gemm_bf16": "video_audio_gen_amd/csrc/gemm.hip",
                 "gemm_mx8": "video_audio_gen_amd/csrc/gemm.hip", "gemm_mx4": "video_audio_gen_amd/csrc/gemm.hip",
                 "attention_bf16": "video_audio_gen_amd/csrc/attention.hip"}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain
    copy's reading), or None when there is none or the kernel's source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    src = KERNEL_SOURCE.get(kernel)
    if src is None or not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for ln in f:
            if ln.startswith("traffic_json: "):
                rec = json.loads(ln[len("traffic_json: "):])
    if rec is None or rec.get("source_sha256_16") != _source_digest(os.path.join(ROOT, src)):
        return None
    return rec.get("bytes_per_launch")


def gemm_shapes(cfg, blocks=True, islands=True):
    """(M, N, K) of the GEMM launches of one forward, in launch order."""
    N = cfg.n_tokens
    D, F = cfg.hidden, cfg.ffn
    out = []
    if cfg.io and islands:
        for s in cfg.segments:
            out.append((s.n_tokens, D, cfg.modalities[s.modality].token_width))
    if blocks:
        for _ in range(cfg.n_blocks):
            out += [(N, 3 * D, D), (N, D, D), (N, 2 * F, D), (N, D, F)]
    if cfg.io and islands:
        for s in cfg.segments:
            out.append((s.n_tokens, cfg.modalities[s.modality].token_width, D))
    return out


def family_work(cfg, split_groups=None):
    """Algorithmic work of one forward per kernel family: (amount, unit).

    GEMM and attention count flops (2MNK; 4*hd*H*sum L_d^2); the bandwidth-bound
    kernels count the bytes they must move once (inputs read + outputs written).
    In the fp32 stream a GEMM result reaches the row kernel after it as fp64
    split-K partials, which that kernel must read: `split_groups(n, k)` gives
    (s_lo, s_hi, col_split), columns below col_split in s_lo splits, and a
    group of one split arrives finished as 4-byte floats; int8 slices are 5
    bytes per value."""
    N, D, F, H, hd = cfg.n_tokens, cfg.hidden, cfg.ffn, cfg.n_heads, cfg.head_dim
    es = 2 if cfg.stream == "bf16" else 4
    L = cfg.n_blocks
    w_es = es
    blocks = sum(2.0 * m * n * k for m, n, k in gemm_shapes(cfg, islands=False))
    islands = sum(2.0 * m * n * k for m, n, k in gemm_shapes(cfg, blocks=False))
    out = {
        # block GEMMs run in the stream dtype; the projections in and out are fp32
        "gemm_bf16": (blocks if cfg.stream == "bf16" and cfg.gemm == "stream" else 0.0, "flop"),
        "gemm_mx8": (blocks if cfg.gemm == "mxfp8" else 0.0, "flop"),
        "gemm_mx4": (blocks if cfg.gemm == "mxfp4" else 0.0, "flop"),
        # MX models: the MLP-out GEMM's input m re-quantized once per block (bf16
        # read, E4M3 + one scale byte per 32 written); h, o, h2 come quantized
        # from their producers
        "quantize_mx8": ((L * N * F * (2 + 1 + 1 / 32)) if cfg.gemm in ("mxfp8", "mxfp4") else 0.0, "byte"),
        "gemm_f32": ((islands if cfg.stream == "bf16" else blocks + islands), "flop"),
        "attention": (attention_flops(cfg), "flop"),
        # x read (f32) + h written: the first block's attention norm (every
        # later norm runs fused with the gated residual before it), plus the
        # final fp32 norm with io
        "modnorm": ((N * D * (4 + es) if L else 0) + (N * D * 8 if cfg.io else 0), "byte"),
        # gated residual + the next norm: x and a read, x and h written; per
        # block the MLP's norm, and every block but the last the next block's
        # attention norm
        "resid_modnorm": ((2 * L - 1) * N * D * (12 + es) if L else 0, "byte"),
        "rope_split": (L * N * (6 * D * es + cfg.rot_dim * 4), "byte"),
        "silu_gate": (L * N * 3 * F * es, "byte"),
        # the last block's closing gated residual (the others are fused)
        "gated_residual": (N * D * 12 if L else 0, "byte"),
        "adaln": (L * cfg.n_mod * 6 * D * cfg.cond_dim * w_es, "byte"),
    }
    if cfg.stream == "f32" and split_groups is not None:
        def part_bytes(n, k):  # one GEMM result [N, n] as its consumer reads it
            s_lo, s_hi, cb = split_groups(n, k)
            per = lambda sp: 4 if sp == 1 else 8 * sp
            return N * (cb * per(s_lo) + (n - cb) * per(s_hi))
        nd = N * D
        # rope_part: partials of q|k|v in, q, k, v out, cos/sin rows
        out["rope_split"] = (L * (part_bytes(3 * D, D) + 3 * nd * 4 + N * cfg.rot_dim * 4), "byte")
        # residual (fp64) read + written, partials in, slices out; the prologue
        # reads x and slices it; with io the last one stores the fp32 norm instead
        rn = L * (part_bytes(D, D) + part_bytes(D, F) + 2 * 16 * nd + 2 * 5 * nd) + (8 * nd + 5 * nd if L else 0)
        out["resid_norm_slice"] = (rn, "byte")
        out["silu_slice"] = (L * (part_bytes(2 * F, D) + 5 * N * F), "byte")
        # slice_rows of each attention output (fp32 in, slices out); the residual
        # widened on entry and, without io, narrowed on exit; with io the slices
        # of the in-projection's tokens and of the final norm
        conv = L * 9 * nd + 12 * nd
        if cfg.io:
            conv += 9 * nd + sum(9 * sg.n_tokens * cfg.modalities[sg.modality].token_width for sg in cfg.segments)
        else:
            conv += 12 * nd
        out["convert"] = (conv, "byte")
    return out


def attention_flops(cfg):
    per_block = 4 * cfg.head_dim * cfg.n_heads * sum(s.n_tokens ** 2 for s in cfg.segments)
    return per_block * cfg.n_blocks


def cpu_baseline(cfg, weights_fn, islands, inp, sample_blocks: int, log=log, min_seconds: float = 10.0):
    """Time the oracle's block forward on this workload's tokens, cycling over the
    weights of `sample_blocks` blocks until at least `min_seconds` of CPU work
    (at least one pass), and scale the per-block time to a forward."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    mode = "bf16" if cfg.stream == "bf16" else "fp64"
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    if cfg.cond_kind == "timestep" and "t" not in inp:
        emb = O.cond_embeddings(cfg, O.denoise_step_conditions(cfg, 0)[0])
    elif cfg.cond_kind == "timestep":
        emb = O.cond_embeddings(cfg, [float(inp["t"][r.source]) for r in cfg.cond_rows])
    else:
        emb = O.cond_embeddings(cfg, None, inp["cond"])
    x = np.random.default_rng(0).standard_normal((cfg.n_tokens, cfg.hidden))
    ws = [weights_fn(b) for b in range(sample_blocks)]
    t0 = time.perf_counter()
    run = 0
    while True:
        b = run % sample_blocks
        mod = O.adaln_table(cfg, ws[b], b, emb, mode)
        x = O.block_forward(cfg, x, mod, ws[b], b, lay, cos, sin, mode, threads=min(cores, 16))
        run += 1
        dt = time.perf_counter() - t0
        if run >= sample_blocks and dt >= min_seconds:
            break
    per_forward = dt / run * cfg.n_blocks
    log(f"cpu oracle: {run} block forwards in {dt:.2f}s -> {per_forward:.2f}s per forward")
    return {"value": cfg.n_tokens / per_forward, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{run} block forwards over the weights of {sample_blocks} of {cfg.n_blocks} blocks "
                      f"({mode}, numpy/OpenBLAS, {cfg.n_tokens} tokens), {dt:.1f}s, scaled to one "
                      f"{cfg.n_blocks}-block forward ({per_forward:.1f}s)"}


def cpu_whole_forward(cfg, inp, log=log):
    """Time one whole forward of the oracle (every block, the projections in
    and out) on one host thread, the way the pages time their host reference
    (page "the 2.4B fp32 DiT onto the device, staged once", section "Speed":
    a single-threaded CPU forward).  The block weights are generated before the
    clock starts."""
    import numpy as np
    import oracle as O
    import synthetic as S
    from threadpoolctl import threadpool_limits

    t0 = time.perf_counter()
    ws = [S.block_weights(cfg, b, threads=8) for b in range(cfg.n_blocks)]
    isl = S.island_weights(cfg) if cfg.io else None
    log(f"cpu oracle: generated {cfg.n_blocks} blocks of weights in {time.perf_counter() - t0:.1f}s")
    with threadpool_limits(1):
        t0 = time.perf_counter()
        out = O.forward(cfg, lambda b: ws[b], isl, inp, threads=1)
        dt = time.perf_counter() - t0
    assert all(np.isfinite(v).all() for v in out.values())
    log(f"cpu oracle: one whole {cfg.n_blocks}-block forward on one thread in {dt:.2f}s")
    return {"value": cfg.n_tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"one whole {cfg.n_blocks}-block forward with the in/out projections (fp64 numpy, "
                      f"one thread, {cfg.n_tokens} tokens): {dt:.2f}s"}


def measure(cfg, steps, warmup, no_graph=False, protocol_loops=5):
    """Stage `cfg`'s weights, time `steps` forwards (or denoise steps) after
    `warmup`, then a per-kernel pass; returns the measurements and the runner."""
    import numpy as np
    import torch

    import synthetic as S  # noqa: F401
    import harness
    from video_audio_gen_amd import dit

    dev = torch.cuda.get_device_name(0)
    log(f"workload {cfg.name}: {cfg.n_blocks} blocks, hidden {cfg.hidden}, {cfg.n_tokens} tokens on {dev}")
    t0 = time.time()
    model = harness.stage_model(cfg, threads=16, log=log)
    log(f"staged {model.weight_bytes / 1e9:.2f} GB of weights in {time.time() - t0:.1f}s")
    r = harness.Runner(cfg, model=model)
    torch.cuda.synchronize()

    # A timestep-conditioned denoise configuration times Euler steps of its
    # schedule (dit_denoise_loop: forward + update per step, latents resident);
    # every other configuration times forwards.
    loop = cfg.denoise_steps > 0 and cfg.cond_kind == "timestep"
    if loop:
        sched = [dit.dit_sigma_schedule(cfg.shifts[m], cfg.denoise_steps) for m in range(cfg.n_mod)]
        conds, dts = [], []
        for i in range(cfg.denoise_steps):
            t_rows = np.asarray([sched[rw.modality][0][i] for rw in cfg.cond_rows], np.float32)
            conds.append(dit.dit_timestep_embedding(t_rows, cfg.cond_dim))
            dts.append([sched[m][1][i] for m in range(cfg.n_mod)])
        cond_tab = torch.from_numpy(np.stack(conds)).cuda()
        dt_tab = torch.from_numpy(np.asarray(dts, np.float32)).cuda()
        lat = r.x_in.clone()
        state = {"i": 0}

        def run_steps(k):
            """k consecutive steps of the schedule; back to the initial noise at step 0."""
            while k > 0:
                i = state["i"]
                if i == 0:
                    lat.copy_(r.x_in)
                n = min(k, cfg.denoise_steps - i)
                dit.dit_denoise_loop(model, r.batch, lat, cond_tab[i:], dt_tab[i:], n, r.ws)
                state["i"] = (i + n) % cfg.denoise_steps
                k -= n
        r.forward = lambda: run_steps(1)

    for _ in range(warmup):
        r.forward()
    torch.cuda.synchronize()
    log(f"warmup {warmup} done")
    # One forward captured by the library as a HIP graph (dit_forward_graph_create:
    # the few hundred launches of the music model replay as one); its output is
    # checked against the eager forward before timing.
    step = r.forward
    if not no_graph and not loop:
        eager = r.forward().clone()
        torch.cuda.synchronize()
        graph = dit.ForwardGraph(r.model, r.batch, r.x_in, r.cond, r.out, r.ws)
        graph.launch()
        torch.cuda.synchronize()
        if not torch.equal(r.out, eager):
            log("graph replay differs from the eager forward; timing eager launches")
        else:
            step = graph.launch
            log(f"timing replays of one captured forward graph ({graph.nodes} nodes)")

    # timed region: exactly K forwards between two synchronisations
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    if loop:
        run_steps(steps)
    else:
        for _ in range(steps):
            step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    log(f"timed {steps} {'denoise steps' if loop else 'forwards'}: {ms:.3f} ms per "
        f"{'step' if loop else 'forward'} (host wall {wall * 1e3 / steps:.3f} ms)")

    # The pages' protocol beside it: loops of R = 1 and R = 3 forwards, each
    # between two events, five of each; median / min / max per forward and the
    # slope over R (the intercept is a loop's fixed cost).
    timing = None
    if not loop and protocol_loops > 0:
        per = {1: [], 3: []}
        for _ in range(protocol_loops):
            for R in (1, 3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(R):
                    step()
                e1.record()
                torch.cuda.synchronize()
                per[R].append(e0.elapsed_time(e1))
        med = {R: float(np.median(v)) for R, v in per.items()}
        slope = (med[3] - med[1]) / 2
        timing = {"loops": protocol_loops,
                  "r1_ms": {"median": round(med[1], 4), "min": round(min(per[1]), 4), "max": round(max(per[1]), 4)},
                  "r3_ms_per_forward": {"median": round(med[3] / 3, 4), "min": round(min(per[3]) / 3, 4),
                                        "max": round(max(per[3]) / 3, 4)},
                  "slope_ms_per_forward": round(slope, 4), "intercept_ms": round(med[1] - slope, 4)}
        log(f"R=1 median {med[1]:.3f} ms, R=3 median {med[3] / 3:.3f} ms per forward, slope {slope:.3f} ms, "
            f"intercept {med[1] - slope:.3f} ms")

    # per-kernel device time: HIP events recorded around every launch on its stream
    dit.dit_profile_begin()
    if loop:
        run_steps(steps)
    else:
        for _ in range(steps):
            r.forward()
    prof = dit.dit_profile_end()
    total_dev = sum(v[1] for v in prof.values())
    for k, (n, t) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        if n:
            log(f"  {k:16s} launches {n:6d}  total {t:9.3f} ms  avg {t / n * 1e3:9.2f} us  "
                f"share {t / total_dev * 100:5.1f}%")
    work = family_work(cfg, dit.dit_gemm_split_groups if cfg.stream == "f32" else None)
    kernels = {}
    for k, (n, t) in prof.items():
        if not n:
            continue
        key = k if k.startswith("gemm") else k.split("_bf16")[0].split("_f32")[0]
        if key not in work or t <= 0:
            continue
        amt, unit = work[key]
        rate = amt * steps / (t * 1e-3)
        if unit == "byte":
            kernels[k] = {"GB/s": round(rate / 1e9, 1), "frac_hbm": round(rate / 1e9 / PEAK["hbm_gbs"], 4),
                          "avg_us": round(t / n * 1e3, 2)}
        else:
            peak = (PEAK["mfma_i8_slices"] if k == "gemm_f32" else PEAK["mfma_fp8"] if k in ("gemm_mx8", "gemm_mx4")
                    else PEAK["mfma_bf16"] if k.endswith("bf16") else None)
            kernels[k] = {"TFLOP/s": round(rate / 1e12, 2), "avg_us": round(t / n * 1e3, 2)}
            if peak:
                kernels[k]["frac_mfma"] = round(rate / 1e12 / peak, 4)
        log(f"  {k:16s} {kernels[k]}")
    fam = max(prof.items(), key=lambda kv: kv[1][1])[0]
    n_launch, fam_ms = prof[fam]
    if fam in ("gemm_f32", "gemm_bf16", "gemm_mx8", "gemm_mx4"):
        flops = work[fam][0] * steps
        peak_key, peak_note = GEMM_FAMILY_PEAK[fam]
        achieved = flops / (fam_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK[peak_key], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK[peak_key], 4), "traffic": None, "kernel": fam,
                "launches": n_launch, "avg_launch_us": round(fam_ms / n_launch * 1e3, 2), "peak_kind": peak_note}
        if fam == "gemm_f32":
            # the same rate against the published fp32 MFMA peak (the unit an fp32 GEMM would otherwise use)
            roof["frac_of_fp32_mfma_peak"] = round(achieved / PEAK["mfma_f32"], 4)
    elif fam == "attention_bf16":
        flops = attention_flops(cfg) * steps
        achieved = flops / (fam_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK["mfma_bf16"], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK["mfma_bf16"], 4), "traffic": None, "kernel": fam,
                "launches": n_launch, "avg_launch_us": round(fam_ms / n_launch * 1e3, 2)}
    else:
        roof = {"bound": "unknown", "achieved": None, "peak": None, "unit": None, "frac": None,
                "traffic": None, "kernel": fam}
    roof["traffic"] = measured_traffic(fam, cfg.name)

    return {"ms": ms, "timing": timing, "kernels": kernels, "roofline": roof, "loop": loop,
            "launch": "hip_graph" if step is not r.forward else "eager", "dev": dev, "runner": r,
            "model": model}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=4)
    ap.add_argument("--cpu-sampled", action="store_true",
                    help="time the oracle on a few blocks with all host threads and scale to a forward "
                         "(the default for an fp32 workload is one whole forward on one thread)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device five times (the known-size kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters), then exit")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every kernel from the host instead of replaying one captured HIP graph")
    ap.add_argument("--extra", default="c4,c4_mxfp8,c4_mxfp4",
                    help="comma-separated workloads timed after the headline one, each in its own timed "
                         "region, reported under their own keys ('none' for none)")
    ap.add_argument("--extra-steps", type=int, default=5)
    ap.add_argument("--extra-warmup", type=int, default=1)
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the path runs on a single device; "
              "multi-GPU sharding is designed, not built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if a.copy_calibration:
        n = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {a.copy_calibration} MiB x 5")
        return 0

    import synthetic as S

    cfg = S.get_config(a.workload)
    res = measure(cfg, a.steps, a.warmup, a.no_graph)
    r, ms, loop, dev = res["runner"], res["ms"], res["loop"], res["dev"]
    timing, kernels, roof = res["timing"], res["kernels"], res["roofline"]

    cpu = None
    if not a.no_cpu_baseline:
        import oracle  # noqa: F401
        if cfg.stream == "f32" and not a.cpu_sampled:
            cpu = cpu_whole_forward(cfg, r.inp)
        else:
            cpu = cpu_baseline(cfg, lambda b: S.block_weights(cfg, b, threads=8), None, r.inp,
                               min(a.cpu_sample_blocks, cfg.n_blocks))

    tokens = cfg.n_tokens
    line = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.stream == "f32" else "bf16",
        "data": "synthetic (seeded; weights N(0,0.02), random init)",
        "config": {"workload": cfg.name, "n_blocks": cfg.n_blocks, "hidden": cfg.hidden,
                   "heads": cfg.n_heads, "head_dim": cfg.head_dim, "ffn": cfg.ffn,
                   "tokens": tokens, "documents": [s.n_tokens for s in cfg.segments],
                   "device": dev, "launch": res["launch"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "timing": timing,
        "kernels": kernels,
    }
    # further workloads after the headline one (the headline model is freed first)
    extras = [w for w in a.extra.split(",") if w and w != "none" and S.get_config(w).name != cfg.name]
    if extras:
        del r, res
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        line["extra"] = {}
        for w in extras:
            ecfg = S.get_config(w)
            e = measure(ecfg, a.extra_steps, a.extra_warmup, a.no_graph, protocol_loops=0)
            line["extra"][w] = {
                "workload": ecfg.name, "dtype": "f32" if ecfg.stream == "f32" else (ecfg.gemm if ecfg.gemm != "stream" else "bf16"),
                "ms_per_forward" if not e["loop"] else "ms_per_step": round(e["ms"], 4),
                "tokens_per_s": round(ecfg.n_tokens / (e["ms"] * 1e-3), 2),
                "steps": a.extra_steps, "warmup": a.extra_warmup, "launch": e["launch"],
                "n_blocks": ecfg.n_blocks, "tokens": ecfg.n_tokens,
                "documents": [sg.n_tokens for sg in ecfg.segments],
                "roofline": e["roofline"], "kernels": e["kernels"]}
            del e
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    if loop:
        line["config"]["denoise_steps"] = cfg.denoise_steps
        line["config"]["timed"] = f"{a.steps} Euler steps of the {cfg.denoise_steps}-step schedule (forward + update each)"
        line["loop_s"] = round(ms * cfg.denoise_steps / 1e3, 3)
        line["loop_s_kind"] = "measured" if a.steps == cfg.denoise_steps else \
            f"{cfg.denoise_steps} x the measured per-step time"
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
