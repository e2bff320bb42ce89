"""The fixed draft-id gate of the bf16 GPU parity tests (CPU).

The gate comes from tests/golden/bf16_noise_floor.txt, which
tests/golden/bf16_noise_floor.py writes from the oracle alone: the oracle in
float64 against the same steps in float32 arithmetic, both rounding to bf16
at the device's storage points.  Checked here: the file covers every bf16
drafter family the GPU tests use, the small family's floor is reproduced by
re-running the script's own comparison (float32 BLAS results may differ in
the last bits between machines, so within a factor of two), and the
float32 evaluation really rounds to bf16 where the float64 oracle does.
"""
import os
import sys

import numpy as np
import pytest

import oracle.dflash_oracle as OD
from block_diffusion_drafter_concat_amd import configs

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import bf16_noise_floor as NF  # noqa: E402

from gpu_util import bf16_noise_floor, id_gate, small_bf16_shape  # noqa: E402


def test_floor_file_covers_every_bf16_family():
    for shape in (small_bf16_shape(), configs.SMALL_D64_BF16, configs.QWEN3_8B_LIKE,
                  configs.TARGET_27B_LIKE, configs.MAX_HIDDEN_BF16):
        f = bf16_noise_floor(shape)
        assert 1e-4 < f < 0.2, (shape, f)
        assert id_gate(shape) == max(1e-2, 2 * f)
    assert id_gate(configs.TINY_F32) == 1e-2


@pytest.mark.parametrize("family", ["small-bf16", "small-bf16-d64"])
def test_small_family_floor_reproduces(family):
    want = bf16_noise_floor(small_bf16_shape() if family == "small-bf16"
                            else configs.SMALL_D64_BF16)
    got = 0.0
    for fam, _, shape, wid, lens, B in NF.cases():
        if fam != family:
            continue
        w = configs.make_weights(shape, wid)
        caches = NF.synthetic_cache(shape, wid, lens)
        anchors = configs.make_anchors(shape, wid, len(lens))
        got = max(got, NF.floor_of(shape, w, caches, anchors, B)["dz"])
    assert want / 2 <= got <= 2 * want, (got, want)


def test_float32_evaluation_keeps_the_rounding_points():
    """Inside float32_arithmetic() the oracle's arrays are float32 and its
    bf16 rounding still lands on bf16 values; outside, float64 is restored."""
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -7.1], dtype=np.float64)
    ref = OD.bf16_round(x)
    assert ref[0] == 1.0 and ref[1] == 1.0 + 2.0 ** -6     # both halfway: ties to even
    with NF.float32_arithmetic():
        assert OD._f64(x).dtype == np.float32
        r = OD.bf16_round(x)
        assert r.dtype == np.float32
        np.testing.assert_array_equal(r.astype(np.float64), ref)
    assert OD._f64(x).dtype == np.float64
    assert OD.bf16_round(x).dtype == np.float64
