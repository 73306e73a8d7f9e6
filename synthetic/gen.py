"""Seeded synthetic weights and inputs.

Every tensor has its own generators, keyed by (seed, key, FNV-1a-64 of the
tensor's name, chunk index) with one PCG64 stream per 4M-value chunk, so any
one tensor -- one block's weights, one segment's latent -- can be regenerated
alone, in any order, on any machine, by any number of threads (numpy's PCG64
and its normal sampler are platform independent).  This follows the pages' practice of
rebuilding weights on both sides of a check from one keyed generator instead of
storing them (page "port the MiniMax-H3 omni-modal video+audio DiT", section
"How this is gated").

Distributions: weights N(0, 0.02^2), biases 0, tokens and latents N(0, 1),
timesteps U(0, 1), conditioning vectors N(0, 1).  For a bf16 stream the block
weights and the token inputs are rounded to the nearest bf16 (ties to even) and
kept as float32 arrays holding bf16-representable values, so both sides receive
identical numbers; ``bf16_bits`` gives their 16-bit encoding.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Tuple

import numpy as np

from .configs import DitConfig

WEIGHT_STD = 0.02


def fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for b in s.encode("utf-8"):
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def tensor_rng(seed: int, key_id: int, name: str) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), int(key_id), fnv1a64(name)])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bf16 value, ties to even, in place."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    u = a.reshape(-1).view(np.uint32)
    step = 1 << 24
    for i in range(0, u.size, step):
        c = u[i:i + step]
        lsb = (c >> np.uint32(16)) & np.uint32(1)
        c += np.uint32(0x7FFF) + lsb
        c &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """16-bit bf16 encoding of a float32 array whose values are bf16-representable."""
    assert a.dtype == np.float32
    u = np.ascontiguousarray(a).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        a *= np.float32(std)
    return a


CHUNK = 1 << 22  # values per independent stream of a large tensor
_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def _keyed_normal(seed: int, key: int, name: str, shape, std: float, bf16: bool) -> np.ndarray:
    """N(0, std^2) float32 values of one tensor.  Value i comes from stream
    (seed, key, name, i // CHUNK), so the result does not depend on how many
    threads fill it; chunks are filled in parallel (numpy releases the GIL)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        ss = np.random.SeedSequence([int(seed), int(key), fnv1a64(name), c])
        g = np.random.Generator(np.random.PCG64(ss))
        g.standard_normal(size=hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)
        if bf16:
            round_to_bf16(out[lo:hi])

    chunks = (n + CHUNK - 1) // CHUNK
    if chunks <= 1:
        fill(0)
    else:
        list(_pool().map(fill, range(chunks)))
    return out.reshape(shape)


def block_weight_shapes(cfg: DitConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """(name suffix, shape) of one block's tensors, nn.Linear layout [out, in]."""
    D, F, dt = cfg.hidden, cfg.ffn, cfg.cond_dim
    out = []
    for m in range(cfg.n_mod):
        out.append((f"adaln.{m}.weight", (6 * D, dt)))
        out.append((f"adaln.{m}.bias", (6 * D,)))
    out += [("attn.qkv.weight", (3 * D, D)), ("attn.qkv.bias", (3 * D,)),
            ("attn.out.weight", (D, D)), ("attn.out.bias", (D,)),
            ("mlp.in.weight", (2 * F, D)), ("mlp.in.bias", (2 * F,)),
            ("mlp.out.weight", (D, F)), ("mlp.out.bias", (D,))]
    return out


def island_weight_shapes(cfg: DitConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """(name, shape) of the fp32 in/out projections, one pair per modality."""
    if not cfg.io:
        return []
    D = cfg.hidden
    out = []
    for m, mod in enumerate(cfg.modalities):
        c = mod.token_width
        out += [(f"in.{m}.weight", (D, c)), (f"in.{m}.bias", (D,)),
                (f"out.{m}.weight", (c, D)), (f"out.{m}.bias", (c,))]
    return out


def _make(cfg: DitConfig, name: str, shape, seed: int, stream_bf16: bool) -> np.ndarray:
    if name.endswith(".bias"):
        return np.zeros(shape, np.float32)
    return _keyed_normal(seed, 1000 + cfg.model_id, name, shape, WEIGHT_STD, stream_bf16)


def block_weights(cfg: DitConfig, b: int, seed: int = 0, threads: int = 1) -> Dict[str, np.ndarray]:
    """One block's weights, keyed 'blocks.{b}.<suffix>'.  (``threads`` is
    accepted for compatibility; large tensors always fill in parallel chunks.)"""
    bf = cfg.stream == "bf16"
    items = [(f"blocks.{b}.{s}", shp) for s, shp in block_weight_shapes(cfg)]
    return {n: _make(cfg, n, shp, seed, bf) for n, shp in items}


def island_weights(cfg: DitConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    return {n: _make(cfg, n, s, seed, False) for n, s in island_weight_shapes(cfg)}


def all_weights(cfg: DitConfig, seed: int = 0, threads: int = 1) -> Dict[str, np.ndarray]:
    w = island_weights(cfg, seed)
    for b in range(cfg.n_blocks):
        w.update(block_weights(cfg, b, seed, threads))
    return w


def segment_latent_shape(cfg: DitConfig, seg_index: int) -> Tuple[int, ...]:
    seg = cfg.segments[seg_index]
    mod = cfg.modalities[seg.modality]
    if mod.io == "patch3d":
        t, h, w = seg.grid
        pt, ph, pw = mod.patch
        return (mod.channels, t * pt, h * ph, w * pw)
    if mod.io == "channel_major":
        return (mod.channels, seg.n_tokens)
    raise ValueError("segment has no latent")


def inputs(cfg: DitConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """The forward's inputs.

    'x'           [N, D] tokens (configurations without in/out projections)
    'latent.{i}'  latent of segment i, [C, T*pt, H*ph, W*pw] or [C, L] (with projections)
    't'           [n_requests] timesteps (timestep conditioning, not the denoise loop)
    'cond'        [n_sources, cond_dim] conditioning vectors (vector conditioning)
    """
    out: Dict[str, np.ndarray] = {}
    k = cfg.key_id
    if cfg.io:
        for i in range(len(cfg.segments)):
            src = i % (len(cfg.segments) // 2) if cfg.cfg_replicate_latent else i
            out[f"latent.{i}"] = _keyed_normal(seed, k, f"latent.{src}", segment_latent_shape(cfg, i), 1.0, False)
    else:
        out["x"] = _keyed_normal(seed, k, "x", (cfg.n_tokens, cfg.hidden), 1.0, cfg.stream == "bf16")
    if cfg.cond_kind == "timestep":
        if cfg.denoise_steps == 0:
            out["t"] = tensor_rng(seed, k, "t").random(cfg.n_requests, dtype=np.float32)
    else:
        n_src = 1 + max(r.source for r in cfg.cond_rows)
        out["cond"] = _normal(tensor_rng(seed, k, "cond"), (n_src, cfg.cond_dim), 1.0)
    return out


def cond_steps(cfg: DitConfig, n_steps: int, seed: int = 0) -> np.ndarray:
    """Per-step conditioning vectors of a vector-conditioned denoise loop,
    [n_steps, n_sources, cond_dim] float32, N(0, 1); step 0 equals
    ``inputs(cfg)['cond']``."""
    n_src = 1 + max(r.source for r in cfg.cond_rows)
    out = np.empty((n_steps, n_src, cfg.cond_dim), np.float32)
    for i in range(n_steps):
        name = "cond" if i == 0 else f"cond.step{i}"
        out[i] = _normal(tensor_rng(seed, cfg.key_id, name), (n_src, cfg.cond_dim), 1.0)
    return out
