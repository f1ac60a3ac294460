"""The torch input encoders in synth (used for tensors drawn on the device)
give the same bytes as synth's NumPy encoders.

Input preparation only: the configurations draw the indexer's q and keys as
N(0, 1) and quantize them (fp8 E4M3 with a row scale; MXFP4, E2M1 with an E8M0
scale per 32).  Both sides of every parity test read the encoded bytes, so
these encoders are not part of what is checked; this test only keeps the two
copies of the rule identical.  Run on the CPU with torch CPU tensors.
"""
import numpy as np
import torch

import synth


def _inputs():
    g = np.random.default_rng(7)
    x = (g.normal(size=(64, 128)) * np.exp(3 * g.normal(size=(64, 1)))).astype(np.float32)
    x[0] = 0.0                                   # an all-zero row / block
    x[1, :32] = 0.0
    x[2] = np.exp2(np.arange(-60, 68)).astype(np.float32)          # powers of two
    x[3] = np.nextafter(np.exp2(np.arange(-60, 68)), 0).astype(np.float32)   # just below them
    # MXFP4 midpoints at a block whose amax is 4 (E = 0): 0.25, 0.75, ..., 5
    x[4, :32] = 0.0
    x[4, 0] = 4.0
    x[4, 1:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -5.0]
    # E4M3 midpoints after the row scale (amax 448 -> scale 1)
    x[5] = 0.0
    x[5, :6] = [448.0, 1.0625, 1.1875, -2.0 ** -10, 1.5 * 2.0 ** -9, 460.0]
    x[6] = np.float32(1e-40)                     # subnormal float32 values
    return x


def test_fp8_rows_same_bytes():
    x = _inputs()
    c_np, s_np = synth.quant_fp8_rows(x)
    c_t, s_t = synth.device_quant_fp8_rows(torch.from_numpy(x))
    assert np.array_equal(c_t.numpy(), c_np)
    assert np.array_equal(s_t.numpy(), s_np)


def test_mxfp4_same_bytes():
    x = _inputs()
    p_np, s_np = synth.quant_mxfp4(x)
    p_t, s_t = synth.device_quant_mxfp4(torch.from_numpy(x))
    assert np.array_equal(p_t.numpy(), p_np)
    assert np.array_equal(s_t.numpy(), s_np)
    # batch axes in front
    x3 = x.reshape(4, 16, 128)
    p3, s3 = synth.device_quant_mxfp4(torch.from_numpy(x3))
    assert np.array_equal(p3.numpy().reshape(64, 64), p_np)
