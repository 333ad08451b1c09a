"""The input generator's MXFP4 storage of float32 master weights: valid codes
and E8M0 scales, and every stored value within the format's rounding bound
of its master (CPU)."""
import numpy as np
import torch

from oracle import codecs
from synthetic.gen import quantize_master_mxfp4


def test_mxfp4_storage_bounds():
    g = torch.Generator().manual_seed(7)
    m = torch.randn(64, 256, generator=g) * 0.03
    m[3, :32] = 0.0                     # an all-zero block
    m[5, 40] = 1.0                      # a block with one large value
    packed, scales = quantize_master_mxfp4(m)
    assert packed.shape == (64, 128) and scales.shape == (64, 8)
    v = codecs.mxfp4_decode(packed.numpy(), scales.numpy())
    mm = m.numpy().astype(np.float64)
    blocks = np.abs(mm).reshape(64, 8, 32).max(-1)
    e = scales.numpy().astype(np.int64) - 127
    nz = blocks > 0
    # shared exponent = floor(log2(amax)) - 2: the block maximum lands in [4, 8)
    assert np.all(e[nz] == np.floor(np.log2(blocks[nz])) - 2)
    # rounding to the nearest E2M1 value: |error| <= half the spacing at that
    # magnitude (spacing 0.5 below 2, 1 below 4, 2 above), saturation at 6
    step = np.repeat(np.ldexp(1.0, e), 32, axis=1)
    t = np.abs(mm) / step
    half = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0))
    err = np.abs(v - mm) / step
    sat = t > 6
    assert np.all(err[~sat] <= half[~sat] + 1e-12)
    assert np.all(np.abs(v[sat]) == 6 * step[sat])
    assert np.all(v[3, :32] == 0)
