"""Drive the library with seeded synthetic workloads (tests and benchmark).

Stages a configuration's weights block by block from the keyed generator in
``synthetic/`` (so a 60 GB model never sits in host memory at once), builds the
batch tables and the conditioning rows, and allocates the workspace.  Every
step of the forward itself runs in libdit.so.
"""

from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

from video_audio_gen_amd import dit


def stage_model(cfg, seed: int = 0, threads: int = 8, device: str = "cuda", log=None) -> dit.Model:
    import synthetic as S
    m = dit.Model(cfg, device)
    bf = cfg.stream == "bf16"
    t0 = time.time()
    if cfg.io:
        dit.dit_stage_weights(m, S.island_weights(cfg, seed))

    def gen(b):
        return S.block_weights(cfg, b, seed, threads=2)

    # generate block b+1 while block b is being copied
    with ThreadPoolExecutor(max(1, threads // 2)) as ex:
        futs = [ex.submit(gen, b) for b in range(min(cfg.n_blocks, 2))]
        for b in range(cfg.n_blocks):
            w = futs[b].result()
            if b + 2 < cfg.n_blocks:
                futs.append(ex.submit(gen, b + 2))
            dit.dit_stage_weights(m, w, as_bf16=bf)
            futs[b] = None
            del w
            if log is not None and (b + 1) % 16 == 0:
                log(f"staged {b + 1}/{cfg.n_blocks} blocks ({time.time() - t0:.1f}s)")
    dit.dit_stage_finalize(m)
    return m


def cond_modality(cfg):
    return [r.modality for r in cfg.cond_rows]


def make_batch(model: dit.Model, cfg) -> dit.Batch:
    return dit.Batch(model, cfg.segments, cond_modality(cfg))


def cond_rows(cfg, inp: Dict[str, np.ndarray], t_rows=None) -> np.ndarray:
    """[n_cond, cond_dim] float32 conditioning rows (embedded timesteps or vectors)."""
    if cfg.cond_kind == "timestep":
        if t_rows is None:
            t_rows = [float(inp["t"][r.source]) for r in cfg.cond_rows]
        return dit.dit_timestep_embedding(np.asarray(t_rows, np.float32), cfg.cond_dim)
    return np.stack([inp["cond"][r.source] for r in cfg.cond_rows]).astype(np.float32)


def cond_step_rows(cfg, cond_steps: np.ndarray) -> np.ndarray:
    """[n_steps, n_cond, cond_dim] rows of a vector-conditioned loop from the
    per-step conditioning vectors [n_steps, n_sources, cond_dim]."""
    return np.stack([cond_rows(cfg, {"cond": c}) for c in cond_steps]).astype(np.float32)


def dt_table(cfg, n_steps: Optional[int] = None) -> np.ndarray:
    """[n_steps, n_mod] float32 step sizes from the library's sigma schedule."""
    n = cfg.denoise_steps if n_steps is None else n_steps
    sig = [dit.dit_sigma_schedule(cfg.shifts[m], cfg.denoise_steps)[1] for m in range(cfg.n_mod)]
    return np.asarray([[sig[m][i] for m in range(cfg.n_mod)] for i in range(n)], np.float32)


def pack_input(cfg, inp: Dict[str, np.ndarray]) -> np.ndarray:
    """The forward's input buffer: tokens [N, D] or all segment latents end to end."""
    if not cfg.io:
        return np.ascontiguousarray(inp["x"], np.float32)
    return np.concatenate([inp[f"latent.{i}"].reshape(-1) for i in range(len(cfg.segments))]).astype(np.float32)


def unpack_output(cfg, flat: np.ndarray) -> Dict[str, np.ndarray]:
    import synthetic.gen as G
    if not cfg.io:
        return {"x": flat.reshape(cfg.n_tokens, cfg.hidden)}
    out, off = {}, 0
    for i in range(len(cfg.segments)):
        shp = G.segment_latent_shape(cfg, i)
        n = int(np.prod(shp))
        out[f"latent.{i}"] = flat[off:off + n].reshape(shp)
        off += n
    return out


class Runner:
    """A staged model plus one batch, its workspace and device buffers."""

    def __init__(self, cfg, seed: int = 0, model: Optional[dit.Model] = None, threads: int = 8, log=None):
        import synthetic as S
        self.cfg = cfg
        self.model = model if model is not None else stage_model(cfg, seed, threads, log=log)
        self.batch = make_batch(self.model, cfg)
        self.ws = dit.workspace(self.batch)
        self.inp = S.inputs(cfg, seed)
        self.x_in = torch.from_numpy(pack_input(cfg, self.inp)).cuda()
        self.out = torch.empty_like(self.x_in) if not cfg.io else torch.empty(
            self.batch.latent_floats, dtype=torch.float32, device="cuda")
        self.cond = None
        if cfg.denoise_steps == 0 or cfg.cond_kind == "vector":
            self.cond = torch.from_numpy(cond_rows(cfg, self.inp)).cuda()

    def forward(self, x_in=None, cond=None, out=None):
        dit.dit_forward(self.model, self.batch, self.x_in if x_in is None else x_in,
                        self.cond if cond is None else cond, self.out if out is None else out, self.ws)
        return self.out if out is None else out

    def output_numpy(self, t=None) -> Dict[str, np.ndarray]:
        torch.cuda.synchronize()
        return unpack_output(self.cfg, (self.out if t is None else t).cpu().numpy())
