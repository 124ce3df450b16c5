"""Boundary sweep of the fused decode step (dsa_decode_step) through the C ABI.

Key counts around the tile (16), list (32 per scan workgroup), 128-key
attention chunk and 2,048 top-k edges, k from 1 to the full 2,048 and 1, 2 or
4 query rows: every case is checked against the fp64 oracle at the 1e-4
near-tie band (top-k) and the attention tolerance, bit for bit against the
top-k of the GPU's own scores, and run a second time without stored scores
(the benchmarked form), which must give the same bits.
"""
import itertools

import numpy as np
import pytest
import torch

from sparse_long_context_index_amd import binding, synth
from test_gpu_parity import check_decode, check_same_without_scores, run_decode

pytestmark = pytest.mark.gpu

LKS = (1, 2, 127, 128, 129, 2047, 2048, 2049, 4097)
KS = (1, 7, 2048)
TS = (1, 2, 4)
CASES = [(lk, k, t) for lk, k, t in itertools.product(LKS, KS, TS) if lk >= t]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda", 0)


@pytest.mark.parametrize("Lk,k,T", CASES)
def test_decode_step_boundaries(dev, Lk, k, T):
    cfg = synth.DecodeConfig("sw", L=Lk - T, T=T, k=k, plant_frac=0.01, seed=7 * Lk + 3 * k + T)
    d = synth.decode_inputs(cfg)
    o, idx, S, lse = run_decode(dev, d, Lk, T, k)
    check_decode(d, Lk, T, k, o, idx, S)
    for t in range(T):                          # the set size: min(k, visible keys), -1 padded
        n = min(k, Lk - T + t + 1)
        assert np.all(idx[t, :n] >= 0) and np.all(idx[t, n:] == -1)
    check_same_without_scores(dev, d, Lk, T, k, o, idx, lse)
