"""Write oracle outputs of full-size workloads to tests/golden/.

    python tests/golden/make_samples.py NAME [--threads 6]

NAME is one of the workloads in ``GOLDENS`` below.  Runs only the CPU oracle
(oracle/), once in its reference mode and once as the control arm (fp32 instead
of fp64 GEMM accumulation, same storage points), on the seeded synthetic inputs
of ``synthetic/``.  Nothing here comes from the GPU path.

Writes two files per workload:
  NAME.npz   the reference values, float32 (every output the workload keeps;
             the oracle's outputs are float32-rounded, so this is exact);
  NAME.json  provenance: configuration, segments, which rows are kept, the
             control arm's drift over each kept tensor (max|d|/rms and
             rms(d)/rms), the per-block drift of the residual stream between
             the two arms, and the wall time of each arm.
A GPU test runs the same seeded workload on the device and applies the bf16
parity criterion with the stored control drift.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synthetic as S  # noqa: E402
from synthetic.configs import Segment, scaled  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

# The 64-block model on four small documents of both modalities (io on): the
# full width and depth the benchmark's model has, at a token count the oracle
# finishes in minutes.
C4_DEPTH = scaled(S.get_config("c4"), name="c4_full_depth_small_tokens",
                  segments=(Segment(0, (1, 4, 8), 0), Segment(1, (24,), 1), Segment(0, (2, 2, 4), 2),
                            Segment(1, (40,), 3)))
# The benchmark's packed layouts (18,432 tokens) through the first two blocks of
# the 64-block model's keyed weights.
C4_TOKENS = scaled(S.get_config("c4"), name="c4_full_tokens_2blocks", n_blocks=2)
C5_TOKENS = scaled(S.get_config("c5"), name="c5_full_tokens_2blocks_step0", n_blocks=2)
C3 = S.get_config("c3")


def c3_rows():
    """Complete output rows of the 6144-wide block: both ends of each document
    and the rows either side of 256-query attention tiles and of the 256-row
    GEMM tiles, plus a few seeded interior rows."""
    v0, v1 = 0, 24576          # video document
    a0, a1 = 24576, 26624      # audio document
    rows = {v0, v0 + 1, 255, 256, 257, 511, 512, 8191, 8192, v1 - 257, v1 - 256, v1 - 1,
            a0, a0 + 1, a0 + 255, a0 + 256, a0 + 1023, a0 + 1024, a1 - 2, a1 - 1}
    rng = np.random.default_rng(2024)
    rows |= set(int(r) for r in rng.choice(26624, 12, replace=False))
    return sorted(rows)


GOLDENS = {
    "c3_block_bf16_rows": dict(cfg=C3, rows=c3_rows),
    "c4_full_depth_small_tokens": dict(cfg=C4_DEPTH),
    "c4_full_tokens_2blocks": dict(cfg=C4_TOKENS),
    "c5_full_tokens_2blocks_step0": dict(cfg=C5_TOKENS, step=0),
}


def _drift(ref, ctl):
    r = np.asarray(ref, np.float64)
    d = np.abs(np.asarray(ctl, np.float64) - r)
    rr = float(np.sqrt(np.mean(r * r)))
    return {"rms": rr, "control_max_rel": float(d.max() / rr),
            "control_rms_rel": float(np.sqrt(np.mean(d * d)) / rr)}


def run(name: str, threads: int) -> str:
    spec = GOLDENS[name]
    cfg = spec["cfg"]
    inp = S.inputs(cfg)
    isl = S.island_weights(cfg)
    t_rows = None
    if "step" in spec:
        t_rows, _ = O.denoise_step_conditions(cfg, spec["step"])
    cache = {}

    def weights(b):
        if b not in cache:
            cache.clear()
            cache[b] = S.block_weights(cfg, b)
        return cache[b]

    xs = {"ref": [], "ctl": []}
    meta = {"workload": name, "config": cfg.name, "seed": 0, "oracle_mode": "bf16",
            "n_blocks": cfg.n_blocks, "n_tokens": cfg.n_tokens,
            "segments": [[s.modality, list(s.grid), s.cond_row] for s in cfg.segments],
            "t_rows": t_rows, "tensors": {}, "depth_drift": []}
    outs = {}
    for arm, accum in (("ref", "fp64"), ("ctl", "fp32")):
        t0 = time.time()
        hook = (lambda b, x, arm=arm: xs[arm].append(np.asarray(x, np.float32).copy()))
        outs[arm] = O.forward(cfg, weights, isl, inp, t_rows=t_rows, threads=threads, accum=accum,
                              block_hook=hook)
        meta[f"{arm}_seconds"] = round(time.time() - t0, 1)
        print(f"{name}: {arm} forward {meta[f'{arm}_seconds']:.0f}s", flush=True)
    for b, (xr, xc) in enumerate(zip(xs["ref"], xs["ctl"])):
        d = _drift(xr, xc)
        meta["depth_drift"].append({"blocks": b + 1, "x_control_max_rel": d["control_max_rel"],
                                    "x_control_rms_rel": d["control_rms_rel"]})
    arrays = {}
    rows = spec["rows"]() if "rows" in spec else None
    if rows is not None:
        meta["rows"] = rows
    for k in sorted(outs["ref"]):
        r = np.asarray(outs["ref"][k], np.float64)
        c = np.asarray(outs["ctl"][k], np.float64)
        if rows is not None:
            r, c = r[rows], c[rows]
        assert np.array_equal(r.astype(np.float32).astype(np.float64), r), "outputs are float32 values"
        meta["tensors"][k] = {"shape": list(r.shape), **_drift(r, c)}
        arrays[k] = r.astype(np.float32)
    np.savez_compressed(os.path.join(HERE, f"{name}.npz"), **arrays)
    path = os.path.join(HERE, f"{name}.json")
    with open(path, "w") as f:
        json.dump(meta, f, indent=1)
    return path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("name", choices=sorted(GOLDENS))
    ap.add_argument("--threads", type=int, default=6)
    a = ap.parse_args()
    print(run(a.name, a.threads))
