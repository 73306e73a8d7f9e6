"""Write sampled oracle outputs of a full-size workload to tests/golden/.

    python tests/golden/make_samples.py c3 [--threads 6]

Runs only the CPU oracle (oracle/): once in its reference mode and once as the
control arm (fp32 instead of fp64 GEMM accumulation, same storage points).
Stores, per output tensor: its shape and rms, the control arm's drift over the
whole tensor (max|d|/rms, rms(d)/rms), and 4096 seeded sample positions with
the reference values there.  A GPU test then runs the same seeded workload on
the device and compares it at those positions.  Nothing here comes from the
GPU path.
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

N_SAMPLES = 4096


def run(name: str, threads: int) -> str:
    cfg = S.get_config(name)
    inp = S.inputs(cfg)
    isl = S.island_weights(cfg)
    cache = {}

    def weights(b):
        if b not in cache:
            cache.clear()
            cache[b] = S.block_weights(cfg, b)
        return cache[b]

    t0 = time.time()
    ref = O.forward(cfg, weights, isl, inp, threads=threads)
    t_ref = time.time() - t0
    print(f"{name}: reference forward {t_ref:.0f}s", flush=True)
    t0 = time.time()
    ctl = O.forward(cfg, weights, isl, inp, threads=threads, accum="fp32")
    print(f"{name}: control forward {time.time() - t0:.0f}s", flush=True)

    out = {"config": cfg.name, "seed": 0, "oracle_mode": "bf16" if cfg.stream == "bf16" else "fp64",
           "reference_seconds": round(t_ref, 1), "tensors": {}}
    rng = np.random.default_rng(12345)
    for k in sorted(ref):
        r = np.asarray(ref[k], np.float64)
        c = np.asarray(ctl[k], np.float64)
        rr = float(np.sqrt(np.mean(r * r)))
        d = np.abs(c - r)
        flat = rng.choice(r.size, size=min(N_SAMPLES, r.size), replace=False)
        flat.sort()
        out["tensors"][k] = {
            "shape": list(r.shape), "rms": rr,
            "control_max_rel": float(d.max() / rr),
            "control_rms_rel": float(np.sqrt(np.mean(d * d)) / rr),
            "index": [int(i) for i in flat],
            "value": [float(v) for v in r.reshape(-1)[flat]],
            "control_value": [float(v) for v in c.reshape(-1)[flat]],
        }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{cfg.name}_samples.json")
    with open(path, "w") as f:
        json.dump(out, f)
    return path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("config")
    ap.add_argument("--threads", type=int, default=6)
    a = ap.parse_args()
    print(run(a.config, a.threads))
