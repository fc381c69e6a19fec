"""Seeded random shapes through every path against the oracle, at the parity tolerances: the
forward with and without the key-range split, then the backward with the minimal workspace or
the one that lets the dK/dV work split. Types, head dims, causal / padding, GQA groups, batch
and sequence length are drawn per case (N from 1 to ~3500, ragged); the draws are fixed by the
seed, so a failure names a reproducible case."""
import numpy as np
import pytest

import gpu_util as gu
from gpu_util import log
from scaled_dot_product_fwd_amd import inputs
from test_bwd_gpu import compare_case

pytestmark = pytest.mark.gpu


def draw(i):
    rng = np.random.default_rng([4242, i])
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.45, 0.1]))
    D = int(rng.choice([16, 32, 64, 128, 256], p=[0.1, 0.1, 0.35, 0.35, 0.1]))
    causal = bool(rng.random() < 0.7)
    padded = bool(rng.random() < 0.3)
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 4))
    N = int(rng.choice([rng.integers(1, 300), rng.integers(300, 1500),
                        rng.integers(1500, 3500)], p=[0.4, 0.45, 0.15]))
    return (dtype, D, causal, padded, B, Hq, Hkv, N, bool(rng.random() < 0.5),
            bool(rng.random() < 0.5))


@pytest.mark.parametrize("i", range(40))
def test_random_shape(i):
    dtype, D, causal, padded, B, Hq, Hkv, N, split, split_ws = draw(i)
    tag = "random %d: %s D%d causal%d pad%d B%d Hq%d Hkv%d N%d" % (
        i, dtype, D, causal, padded, B, Hq, Hkv, N)
    log(tag)
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[4243, i])
    O, L = gu.run_device(case, split=split)
    O_ref, L_ref = gu.run_oracle(case)
    gu.compare(case, O, L, O_ref, L_ref, tag="%s split %d" % (tag, split))
    if N * B * Hq <= 300000:   # the oracle's backward in a few seconds
        dout = inputs.make_grad(case, [4243, i])
        compare_case(case, dout, tag + " bwd", split_ws=split_ws)
