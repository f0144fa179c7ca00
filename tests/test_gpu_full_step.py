"""The 30-layer 720P step with planted head behaviour: one-time classification must
recover every planted label (54 Sink / 90 Dummy / 126 Spatial / 90 Global over the
360 (layer, head) pairs), then routed attention runs over all layers with the
recovered labels; sampled rows of three layers are checked against the oracle, with
the bf16 tolerance widened by the outputs' own bf16 storage rounding (planted heads
produce outputs up to |o| ~ 4, where that rounding alone exceeds 1e-2)."""
import numpy as np
import pytest
import torch

from gpu_util import assert_close_bf16_storage, host, sample_rows
from head_routed_sparse_amd import headcast as hc
from head_routed_sparse_amd import inputs as hin
from oracle import headcast_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hc.lib()


def test_full720p_planted_labels_recovered_then_routed():
    cfg = hin.CONFIGS["full720p"]
    g = cfg["geom"]
    desc = hc.make_desc(g)
    params = hc.hc_default_classify_params(gamma=0.5)
    planted = hin.full_step_labels("full720p")
    ws = torch.empty(hc.hc_classify_workspace_bytes(desc, params, g.hist_frames), dtype=torch.uint8, device="cuda")
    got = np.zeros_like(planted)
    margins = []
    check_layers = (0, 15, 29)
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
        # routed attention with the recovered labels
        buf = hc.hc_build_head_buffers(desc, labels, t["k_hist"], t["v_hist"], t["n_hist_frames"])
        out = hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"])
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        if layer in check_layers:
            inp = hin.LayerInputs(g, labels, *(host(t[k]).astype(np.float32) for k in
                                              ("q", "k_hist", "v_hist", "k_cur", "v_cur")), t["n_hist_frames"])
            rows = sample_rows(g, n_random=24, seed=layer)
            want = orc.routed_attention(inp, rows=rows)
            print(layer, assert_close_bf16_storage(host(out)[rows], want, what=f"layer {layer}"))
        del buf, out, t
    assert np.array_equal(got, planted), np.argwhere(got != planted)
    print(f"360/360 labels recovered; smallest margin to a threshold {min(margins):.3f}")
    assert min(margins) >= 0.04
