"""The half-ulp term of the attention tolerance is exactly the output dtype's rounding."""
import numpy as np
import torch

from gpu_helpers import half_ulp


def test_half_ulp_bounds_round_to_nearest_even():
    rng = np.random.default_rng(0)
    # float32 inputs: torch narrows float64 -> float32 -> 16 bit, which would round twice
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 3, 100)]
                       ).astype(np.float32).astype(np.float64)
    for dt in (torch.bfloat16, torch.float16):
        r = torch.from_numpy(x).to(dt).double().numpy()
        err = np.abs(r - x)
        hu = half_ulp(x, dt)
        assert np.all(err <= hu * (1 + 1e-12))
        assert np.max(err / hu) > 0.99          # and the bound is attained, not loose
