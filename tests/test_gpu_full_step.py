"""The 30-layer 720P step with planted head behaviour (54 Sink / 90 Dummy / 126 Spatial
/ 90 Global over the 360 (layer, head) pairs).

* Three whole layers with the seeded numpy inputs: the GPU classification of every
  head (all 10800 queries, the full window) must give the oracle's labels, stored in
  tests/golden/ by make_full720p_golden.py (HeadCast Sec. 4.2, Eqs. 2-5), and its six
  statistics within 3e-3 of the oracle's; then routed attention with those labels on
  sampled rows (>= 512 random rows per head) against the oracle.
* All 30 layers with inputs drawn on the device (fast): classification recovers every
  planted label with every statistic >= 0.04 from its threshold, and routed attention
  runs on every layer with the recovered labels.

Outputs of planted heads concentrate attention on a few keys and reach |o| ~ 3.4; the
output check allows the bf16 tolerance plus the exact half-ulp of storing |o| in bf16
and reports how many elements exceed the plain 1e-2.
"""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import assert_close_bf16_storage, host, sample_rows, to_device
from head_routed_sparse_amd import headcast as hc
from head_routed_sparse_amd import inputs as hin
from oracle import headcast_oracle as orc

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GOLDEN_LAYERS = (0, 15, 29)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hc.lib()


@pytest.mark.parametrize("layer", GOLDEN_LAYERS)
def test_full720p_layer_labels_and_statistics_match_oracle(layer):
    with open(os.path.join(GOLDEN, f"full720p_classify_layer{layer}.json")) as f:
        gold = json.load(f)
    inp = hin.full_step_layer_inputs("full720p", layer)
    g = inp.geom
    t = to_device(inp)
    desc = hc.make_desc(g)
    labels, stats = hc.hc_classify_heads(desc, hc.hc_default_classify_params(gamma=0.5), t["q"], t["k_hist"],
                                         t["v_hist"], inp.n_hist_frames, t["k_cur"], t["v_cur"])
    assert gold["labels"] == gold["planted_labels"]
    assert list(labels) == gold["labels"], (list(labels), gold["labels"])
    diff = np.abs(stats - np.array(gold["stats"]))
    print(f"layer {layer}: labels {list(labels)}, largest statistic difference {diff.max():.2e}")
    assert diff.max() <= 3e-3, diff.max()
    buf = hc.hc_build_head_buffers(desc, labels, t["k_hist"], t["v_hist"], inp.n_hist_frames)
    out = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    rows = sample_rows(g, n_random=512, seed=layer)
    want = orc.routed_attention(inp, labels=labels, rows=rows)
    mx, mean, mag, n_over = assert_close_bf16_storage(out[rows], want, what=f"layer {layer}")
    print(f"layer {layer}: routed max-abs {mx:.3e} (|o| up to {mag:.2f}), mean-abs {mean:.2e}, "
          f"{n_over} of {want.size} elements beyond 1e-2")


def test_full720p_planted_labels_recovered_then_routed():
    cfg = hin.CONFIGS["full720p"]
    g = cfg["geom"]
    desc = hc.make_desc(g)
    params = hc.hc_default_classify_params(gamma=0.5)
    planted = hin.full_step_labels("full720p")
    ws = torch.empty(hc.hc_classify_workspace_bytes(desc, params, g.hist_frames), dtype=torch.uint8, device="cuda")
    got = np.zeros_like(planted)
    margins = []
    for layer in range(cfg["layers"]):
        t = hin.full_step_layer_torch("full720p", layer)
        labels, stats = hc.hc_classify_heads(desc, params, t["q"], t["k_hist"], t["v_hist"], t["n_hist_frames"],
                                             t["k_cur"], t["v_cur"], workspace=ws)
        got[layer] = labels
        for h, lab in enumerate(planted[layer]):
            cs, cd, cp, _, _, sc = stats[h]
            if lab == 0:
                margins.append(cs - 0.95)
            elif lab == 1:
                margins += [0.95 - cs, cd - 0.95]
            elif lab == 2:
                margins += [0.95 - cs, 0.95 - cd, cp - 0.95, sc - 0.755]
            else:
                margins += [0.95 - cs, 0.95 - cd, max(0.95 - cp, 0.755 - sc)]
        buf = hc.hc_build_head_buffers(desc, labels, t["k_hist"], t["v_hist"], t["n_hist_frames"])
        out = hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"])
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        del buf, out, t
    assert np.array_equal(got, planted), np.argwhere(got != planted)
    print(f"360/360 labels recovered; smallest margin to a threshold {min(margins):.3f}")
    assert min(margins) >= 0.04
