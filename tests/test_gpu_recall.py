"""GPU parity of the index-selection recall (dsa_index_recall) through the C ABI.

Bar: the logits are bf16 products summed in fp32 (relative error ~1e-6 of
sum |q k|), and exp2 / log2 are within a few ulp, so each log-sum-exp is off
by well under 1e-5; recall = exp(lse_sel - lse_dense) is checked to 1e-4
relative + 1e-6 absolute.  Cases: random and indexer-chosen sets, every
visible key (recall 1), the empty set (recall 0), several tokens (causal
denominators) and cache rows past Lk NaN-poisoned.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_index_amd import binding, synth

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0
RTOL, ATOL = 1e-4, 1e-6


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda", 0)


def g(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def inputs(T, Lk, seed, extra=0):
    rng = np.random.default_rng(seed)
    q = synth.encode_bf16((rng.standard_normal((T, 64, 192)) * 3).astype(np.float32))
    k = synth.encode_bf16(rng.standard_normal((Lk + extra, 4, 192)).astype(np.float32))
    v = synth.encode_bf16(rng.standard_normal((Lk + extra, 4, 128)).astype(np.float32))
    if extra:
        k[Lk:] = BF16_NAN
        v[Lk:] = BF16_NAN
    return q, k, v


def run(dev, q, k, v, Lk, idx, sm):
    T = q.shape[0]
    lse = torch.empty((T, 64), dtype=torch.float32, device=dev)
    rec = binding.dsa_index_recall(g(q, dev), g(k, dev), g(v, dev), Lk, g(idx.astype(np.int32), dev), sm,
                                   lse_dense=lse)
    torch.cuda.synchronize()
    return rec.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("T,Lk,n", [(1, 5000, 2048), (3, 20000, 700), (2, 2049, 2048), (1, 1, 1), (4, 70000, 2048)])
def test_recall_random_sets(dev, T, Lk, n):
    q, k, v = inputs(T, Lk, seed=T + Lk, extra=5)
    rng = np.random.default_rng(Lk)
    idx = -np.ones((T, n), np.int64)
    for t in range(T):
        vis = Lk - T + t + 1
        m = min(n, vis)
        idx[t, :m] = np.sort(rng.choice(vis, m, replace=False))
    sm = 1 / math.sqrt(192)
    rec, lse = run(dev, q, k, v, Lk, idx, sm)
    rec_ref, lse_ref = oracle.index_recall(q, k, idx, Lk, T, sm)
    assert np.allclose(rec, rec_ref, rtol=RTOL, atol=ATOL), np.max(np.abs(rec - rec_ref))
    assert np.allclose(lse, lse_ref, rtol=1e-5, atol=1e-4)


def test_recall_of_every_visible_key_and_of_none(dev):
    T, Lk = 2, 1500
    q, k, v = inputs(T, Lk, seed=7, extra=3)
    full = np.stack([np.where(np.arange(2048) <= Lk - T + t, np.arange(2048), -1) for t in range(T)])
    rec, _ = run(dev, q, k, v, Lk, full, 0.1)
    assert np.allclose(rec, 1.0, rtol=RTOL)
    rec0, _ = run(dev, q, k, v, Lk, -np.ones((T, 16), np.int64), 0.1)
    assert np.all(rec0 == 0)


def test_recall_of_the_indexer_selection(dev):
    # the decode step's own top-2,048 on the planted 128K verify workload
    cfg = synth.DecodeConfig("r", L=131072, T=2, k=2048, plant_frac=0.005, seed=21)
    d = synth.decode_inputs(cfg)
    Lk = cfg.Lk
    idx = torch.empty((2, 2048), dtype=torch.int32, device=dev)
    binding.dsa_decode_step(g(d["q_idx"], dev), g(d["w"], dev), g(d["k_idx"], dev), g(d["q"], dev), g(d["k"], dev),
                            g(d["v"], dev), Lk, 2, 2048, g(d["sink"], dev), float(d["sm_scale"]), idx_out=idx)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy().astype(np.int64)
    rec, _ = run(dev, d["q"], d["k"], d["v"], Lk, idx_h, float(d["sm_scale"]))
    rec_ref, _ = oracle.index_recall(d["q"], d["k"], idx_h, Lk, 2, float(d["sm_scale"]))
    assert np.allclose(rec, rec_ref, rtol=RTOL, atol=ATOL)
    assert np.all((rec > 0) & (rec < 1))
