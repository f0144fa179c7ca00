"""Helpers shared by the GPU tests: moving seeded inputs to the device and picking
query rows for sampled parity checks."""
import numpy as np
import torch


def dev(a, dtype):
    """float32 numpy array (holding bf16 values for bf16) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def to_device(inp):
    g = inp.geom
    return dict(q=dev(inp.q, g.dtype), k_hist=dev(inp.k_hist, g.dtype), v_hist=dev(inp.v_hist, g.dtype),
                k_cur=dev(inp.k_cur, g.dtype), v_cur=dev(inp.v_cur, g.dtype))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def sample_rows(geom, n_random=256, seed=0):
    """Frame corners, edge midpoints and the centre of every chunk frame, plus random rows."""
    S, fh, fw = geom.tokens_per_frame, geom.frame_h, geom.frame_w
    pts = [(0, 0), (0, fw - 1), (fh - 1, 0), (fh - 1, fw - 1), (0, fw // 2), (fh - 1, fw // 2),
           (fh // 2, 0), (fh // 2, fw - 1), (fh // 2, fw // 2), (1, 1), (fh - 2, fw - 2)]
    rows = {f * S + r * fw + c for f in range(geom.chunk_frames) for r, c in pts if 0 <= r < fh and 0 <= c < fw}
    rng = np.random.default_rng(seed)
    rows |= set(rng.integers(0, geom.lq, size=n_random).tolist())
    return np.array(sorted(rows))


def assert_close(got, want, max_abs, mean_abs, what=""):
    err = np.abs(got - want)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err.max() <= max_abs, f"{what}: max-abs {err.max():.3e} > {max_abs}"
    assert err.mean() <= mean_abs, f"{what}: mean-abs {err.mean():.3e} > {mean_abs}"
    return float(err.max()), float(err.mean())


TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-4, 1e-5)}


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 (8 significant bits) around |x|: 2^(e - 8) for
    |x| in [2^e, 2^(e + 1)); the largest error of storing x in bf16 by rounding to nearest."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def assert_close_bf16_storage(got, want, what=""):
    """The bf16 tolerance (max-abs 1e-2, mean-abs 1e-3) for the kernel's own error, plus
    the exact rounding of a bf16 output: the half-ulp at the larger of |got| and |want|
    (planted heads concentrate attention on a few keys and reach |o| ~ 3.4, where the
    half-ulp is 2^-7 = 7.8e-3; from |o| = 4 on it is 1.6e-2, beyond 1e-2 by itself).
    Returns (max error, mean error, largest |want|, elements beyond the plain 1e-2)."""
    err = np.abs(got - want)
    room = 1e-2 + bf16_half_ulp(np.maximum(np.abs(got), np.abs(want)))
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    bad = err > room
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond 1e-2 + half-ulp (max err {err.max():.3e})"
    assert err.mean() <= 1e-3, f"{what}: mean-abs {err.mean():.3e}"
    return float(err.max()), float(err.mean()), float(np.abs(want).max()), int((err > 1e-2).sum())
