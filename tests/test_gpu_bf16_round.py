"""The device's float32 -> bf16 rounding on every float32 input (needs an MI355X).

Every bf16 value the library stores goes through one of two conversions
(scalar, and pairs packed into 32 bits).  Both are run over all 2^32 float32
bit patterns, in chunks, and compared with torch's own round-to-nearest-even
conversion (a library routine, not this library's code); NaN inputs must give
a NaN.  A sample of the patterns is also compared with the oracle's pinned
definition (oracle.bf16_round).
"""
import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CHUNK = 1 << 28


@pytest.mark.parametrize("packed", [False, True])
def test_bf16_round_every_float32_input(packed):
    import torch
    L.load()
    out = torch.empty(CHUNK, dtype=torch.int16, device="cuda")
    bad = 0
    for c in range((1 << 32) // CHUNK):
        lo = -(1 << 31) + c * CHUNK
        bits = torch.arange(lo, lo + CHUNK, dtype=torch.int32, device="cuda")
        x = bits.view(torch.float32)
        L.debug_bf16_round(x, out, packed=packed)
        ref = x.to(torch.bfloat16).view(torch.int16)
        nan = torch.isnan(x)
        o32 = out.to(torch.int32) & 0xFFFF
        out_nan = ((o32 & 0x7F80) == 0x7F80) & ((o32 & 0x7F) != 0)
        bad += int(((out != ref) & ~nan).sum().item()) + int((nan & ~out_nan).sum().item())
        del bits, x, ref, nan, o32, out_nan
    torch.cuda.synchronize()
    print(f"bf16 rounding ({'pair' if packed else 'scalar'} conversion): {bad} of 2^32 differ",
          flush=True)
    assert bad == 0


def test_bf16_round_matches_oracle_definition():
    import torch
    L.load()
    g = np.random.default_rng(16)
    pats = np.concatenate([
        g.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32),
        # halfway cases (ties to even), subnormals, the largest finite values, +-inf
        (np.arange(0, 1 << 16, dtype=np.uint32) << 16) | np.uint32(0x8000),
        np.arange(0, 1 << 16, dtype=np.uint32),
        np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
                  0x80000000, 0x00000001], dtype=np.uint32)])
    x = pats.view(np.float32)
    x = x[np.isfinite(x) | np.isinf(x)]
    x = x[~np.isnan(x)]
    xd = torch.from_numpy(x.copy()).cuda()
    out = torch.empty(xd.numel(), dtype=torch.int16, device="cuda")
    L.debug_bf16_round(xd, out)
    torch.cuda.synchronize()
    got = (out.cpu().numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    want = O.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got.astype(np.float64), want)
