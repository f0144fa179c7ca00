"""The allocation-free routed call (hc_routed_attention_noalloc, the library's own scratch
instead of a caller workspace) against hc_routed_attention on the same handle state:
two calls in a row, the second with a smaller layer; outputs must be bitwise equal where
both plan the same launches, and within the bf16 tolerance of each other where the
scratch-bounded plan splits the keys differently. Each output is also checked against
the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, assert_close, host, to_device
from head_routed_sparse_amd import headcast as hc
from head_routed_sparse_amd import inputs as hin
from oracle import headcast_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hc.lib()


def one_call(geom, labels, seed, variant=0):
    inp = hin.generate(geom, labels, seed=seed)
    t = to_device(inp)
    buf = hc.hc_build_head_buffers(hc.make_desc(geom, variant), inp.labels, t["k_hist"], t["v_hist"],
                                   inp.n_hist_frames)
    ref = host(hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"]))
    got = host(hc.hc_routed_attention_noalloc(buf, t["q"], t["k_cur"], t["v_cur"]))
    torch.cuda.synchronize()
    return inp, ref, got


def test_noalloc_matches_routed_call_twice_second_smaller():
    big = hin.Geometry(8, 128, 12, 20, 3, 12, 4, 4, "bf16")
    small = hin.Geometry(4, 64, 5, 9, 2, 8, 3, 3, "bf16")
    for geom, labels, seed in ((big, (0, 1, 2, 3, 3, 2, 1, 0), 41), (small, (2, 3, 0, 1), 42)):
        inp, ref, got = one_call(geom, labels, seed)
        assert np.isfinite(got).all()
        assert_close(got, ref, 2e-3, 2e-4, what=f"noalloc vs routed {geom}")
        assert_close(got, orc.routed_attention(inp), *TOL["bf16"], what=f"noalloc vs oracle {geom}")


def test_noalloc_full_size_720p_and_1080p_rows():
    """The benchmark's layers: the scratch-bounded plan (fewer key splits at 1080P) gives
    the routed call's result within rounding order."""
    for name in ("720p", "1080p"):
        cfg = hin.CONFIGS[name]
        g = cfg["geom"]
        t = hin.generate_torch(g, cfg["labels"], 5)
        buf = hc.hc_build_head_buffers(hc.make_desc(g), cfg["labels"], t["k_hist"], t["v_hist"],
                                       t["n_hist_frames"])
        ref = hc.hc_routed_attention(buf, t["q"], t["k_cur"], t["v_cur"])
        got = hc.hc_routed_attention_noalloc(buf, t["q"], t["k_cur"], t["v_cur"])
        got2 = hc.hc_routed_attention_noalloc(buf, t["q"], t["k_cur"], t["v_cur"])
        torch.cuda.synchronize()
        assert torch.equal(got, got2)
        err = (got.float() - ref.float()).abs()
        assert err.max().item() <= 2e-3 and err.mean().item() <= 2e-4, (name, err.max().item())
        del buf, t
