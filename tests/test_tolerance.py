"""The bf16 storage term of the output tolerance, checked against torch's own
float -> bfloat16 rounding (round to nearest even)."""
import numpy as np
import torch

from gpu_util import bf16_half_ulp


def test_half_ulp_bounds_torch_bf16_rounding_tightly():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.3, 1.0, 3.0, 40.0)])
    r = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    err = np.abs(r - x.astype(np.float32).astype(np.float64))
    hu = bf16_half_ulp(x)
    assert np.all(err <= hu * (1 + 1e-12))
    assert np.max(err / hu) > 0.999               # the bound is reached
    # hand values: [1, 2) -> 2^-8, [2, 4) -> 2^-7, [0.5, 1) -> 2^-9, 4 -> 2^-6
    assert list(bf16_half_ulp([1.0, 1.99, 2.0, 3.4, 0.75, 4.0])) == [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7,
                                                                     2.0 ** -9, 2.0 ** -6]
