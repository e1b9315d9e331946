"""Worker for the exhaustive fp8 encoder sweep (runs in spawned processes).

Compares the oracle's e4m3fn encoder with torch's CPU float8_e4m3fn cast over a
contiguous range of fp32 bit patterns.  Kept in its own module so that spawned
workers can import it without importing a test module.
"""
import numpy as np
import torch

from oracle import e4m3fn_encode_rne


def check_range(args):
    lo, hi = args
    torch.set_num_threads(1)
    bits = np.arange(lo, hi, dtype=np.uint32)
    y = bits.view(np.float32)
    mine = e4m3fn_encode_rne(y)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(mine != theirs)[0]
    return int(bad.size), (int(bits[bad[0]]) if bad.size else None)
