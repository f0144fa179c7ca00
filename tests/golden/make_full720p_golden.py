"""Writes tests/golden/full720p_classify_layer<L>.json: the oracle's classification of
whole layers of the 30-layer planted 720P workload (every one of the 10800 queries,
the full 21-frame window).

HeadCast Sec. 4.2: reference output over the full window (Eq. 2), the Sink / Dummy /
Spatial proxies, mean token cosines (Eq. 3), the conservative Spatial score (Eq. 4) and
the decision (Eq. 5); gamma = 0.5 as the workload states. Inputs are the seeded numpy
recipe of head_routed_sparse_amd.inputs.full_step_layer_inputs (PCG64([2607, layer + 1]),
planted heads). Only the oracle computes the stored values.

Usage: python tests/golden/make_full720p_golden.py LAYER [LAYER ...]   (about 10 min per
layer on 8 cores; layers run one after another)
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from head_routed_sparse_amd import inputs as hin  # noqa: E402
from oracle import headcast_oracle as orc  # noqa: E402

PARAMS = dict(gamma=0.5)
KEYS = ("cos_sink", "cos_dummy", "cos_spatial", "p5", "mse", "score")


def golden(layer: int) -> dict:
    inp = hin.full_step_layer_inputs("full720p", layer)
    t0 = time.perf_counter()
    labels, stats = orc.classify_heads(inp, PARAMS)
    dt = time.perf_counter() - t0
    planted = hin.full_step_labels("full720p")[layer]
    g = inp.geom
    return {
        "what": "oracle classification of one whole layer of the planted 30-layer 720P workload "
                "(HeadCast Sec. 4.2, Eqs. 2-5; all query rows, full window)",
        "layer": layer,
        "input_recipe": "head_routed_sparse_amd.inputs.full_step_layer_inputs('full720p', layer): "
                        "numpy PCG64([2607, layer + 1]), N(0,1) Q/K/V then planted vectors, bf16 RNE",
        "geometry": dict(num_heads=g.num_heads, head_dim=g.head_dim, frame_h=g.frame_h, frame_w=g.frame_w,
                         chunk_frames=g.chunk_frames, window_frames=g.window_frames, grid=[g.grid_h, g.grid_w]),
        "params": dict(PARAMS, theta=[0.95, 0.95, 0.95], theta_score=0.755, percentile=5.0),
        "planted_labels": [int(x) for x in planted],
        "labels": [int(x) for x in labels],
        "stats_keys": list(KEYS),
        "stats": [[float(st[k]) for k in KEYS] for st in stats],
        "oracle_seconds": round(dt, 1),
    }


def main():
    for layer in (int(a) for a in sys.argv[1:]):
        rec = golden(layer)
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"full720p_classify_layer{layer}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        agree = rec["labels"] == rec["planted_labels"]
        print(f"layer {layer}: labels {rec['labels']} (planted agree: {agree}), {rec['oracle_seconds']} s",
              flush=True)


if __name__ == "__main__":
    main()
