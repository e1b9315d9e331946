"""Shared helpers for the GPU parity tests (host-side marshalling only)."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Attention tolerance: 2e-3 absolute on the fp32-accumulated result (the PagedAttention
# page's tiny test, whose outputs are fp16 in [-4, 4]), plus half a unit in the last place
# of the output dtype at the oracle's value: the final round-to-nearest-even into bf16 /
# fp16 is part of the specified output and alone reaches 3.9e-3 for bf16 values in [1, 2).
ATTN_TOL = 2e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_45_amd as P
    P.load_library()          # raises if the HIP library is missing: no fallback exists
    return P


def bits16(t: torch.Tensor) -> np.ndarray:
    """fp16/bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def np_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def dtype_name(dt) -> str:
    return "bf16" if dt == torch.bfloat16 else "f16"


def f32_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def half_ulp(want, dtype) -> np.ndarray:
    """Half the spacing of `dtype` (torch.bfloat16 / torch.float16) numbers around |want|."""
    mant, min_exp = (7, -126) if dtype == torch.bfloat16 else (10, -14)
    a = np.maximum(np.abs(want), 2.0 ** min_exp)
    e = np.floor(np.log2(a))
    return 0.5 * np.exp2(e - mant)


def report(tag, got, want, dtype=torch.float16):
    """Prints the raw error statistics; returns the largest error in excess of the output
    dtype's own rounding (compared against ATTN_TOL)."""
    err = np.abs(got.astype(np.float64) - want)
    excess = err - half_ulp(want, dtype)
    msg = (f"{tag}: max_abs_err={err.max():.3e} mean={err.mean():.3e} "
           f"p99={np.quantile(err, 0.99):.3e} max_beyond_output_rounding={excess.max():.3e}")
    print(msg, flush=True)
    return excess.max()
