"""GPU parity of the fused prefill top-k (dsa_prefill_topk) through the C ABI.

The fused call must return, row for row, exactly the index set of the
unfused path on the same GPU arithmetic (dsa_index_scores with T > 8, then
dsa_topk): its threshold and candidate slots may change how the set is found,
never which set it is.  Against the fp64 oracle the set obeys the same top-k
rule as the unfused path (near-tie band of the prefill score bound).  Cases
cover rows that take the threshold, rows whose visible keys all fit, rows
that fall back (every score equal; a run of near-equal winners larger than
the slots), tiny inputs, and the full 8,192 x 1,056,768 chunk on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_index_amd import binding, synth

pytestmark = pytest.mark.gpu

PREFILL_REL = 2.0 ** -10 + 4e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda", 0)


def g(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def unfused(qd, wd, kd, Lk, T, k, r0, r1, ws):
    """Rows r0 .. r1-1 (r1 - r0 >= 9, the contraction's arithmetic) by the
    unfused path: scores of the block of rows, then the top-k of each row."""
    lk = Lk - (T - r1)
    S = binding.dsa_index_scores(qd[r0:r1], wd[r0:r1], kd, lk, r1 - r0)
    idx = binding.dsa_topk(S, lk, r1 - r0, k, ws=ws)
    return idx.cpu().numpy(), S


def check_rows_oracle(d, Lk, T, k, idx_h, rows):
    kf = oracle.decode_e4m3(d["k_idx"])
    kabs = np.abs(kf)
    for r in rows:
        n = Lk - T + r + 1
        qf = oracle.decode_e4m3(d["q_idx"][r])
        S_ref = np.asarray(d["w"][r], np.float64) @ np.maximum(qf @ kf[:n].T, 0.0)
        bound = PREFILL_REL * (np.abs(np.asarray(d["w"][r], np.float64)) @ (np.abs(qf) @ kabs[:n].T)) + 1e-30
        ok, msg = oracle.topk_check(idx_h[r], oracle.topk_row(S_ref, k), S_ref, k, err_bound=bound)
        assert ok, f"row {r}: {msg}"


def run_case(dev, d, Lk, T, k, block=16, oracle_rows=()):
    qd, wd, kd = g(d["q_idx"], dev), g(d["w"], dev), g(d["k_idx"], dev)
    ws = binding.Workspace()
    idx = binding.dsa_prefill_topk(qd, wd, kd, Lk, T, k, ws=ws)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    ws2 = binding.Workspace()
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        a0 = r1 - max(block, 9) if r1 - r0 < 9 else r0     # keep >= 9 rows per unfused call
        a0 = max(a0, 0)
        ref, _ = unfused(qd, wd, kd, Lk, T, k, a0, r1, ws2)
        assert np.array_equal(idx_h[r0:r1], ref[r0 - a0:]), f"rows {r0}..{r1 - 1} differ from the unfused path"
    check_rows_oracle(d, Lk, T, k, idx_h, oracle_rows)
    return idx_h


@pytest.mark.parametrize("L,T,k", [(20000, 64, 2048), (40000, 33, 100), (5000, 40, 2048), (100, 9, 2048),
                                   (300, 12, 7), (70000, 16, 1000)])
def test_prefill_topk(dev, L, T, k):
    cfg = synth.DecodeConfig("p", L=L, T=T, k=k, plant_frac=0.01, seed=L + T)
    d = synth.decode_inputs(cfg, with_kv=False)
    run_case(dev, d, cfg.Lk, T, k, oracle_rows=(0, T - 1))


def test_prefill_topk_all_scores_tie(dev):
    # every score is zero: every long row overflows its slots and falls back
    cfg = synth.DecodeConfig("z", L=20000, T=12, k=2048, plant_frac=0.0, seed=3)
    d = synth.decode_inputs(cfg, with_kv=False)
    d["q_idx"] = np.zeros_like(d["q_idx"])
    idx_h = run_case(dev, d, cfg.Lk, cfg.T, cfg.k)
    for t in range(cfg.T):
        assert np.array_equal(idx_h[t], np.arange(2048))


def test_prefill_topk_clustered_winners(dev):
    # a run of 10,000 near-copies of one row's best key: more winners near
    # the threshold than slots for that row
    cfg = synth.DecodeConfig("c", L=60000, T=10, k=2048, plant_frac=0.0, seed=8)
    d = synth.decode_inputs(cfg, with_kv=False)
    S = oracle.index_scores(d["q_idx"][:1], d["w"][:1], d["k_idx"], cfg.Lk - cfg.T + 1, 1)
    best = int(np.argmax(S[0]))
    rows = np.repeat(d["k_idx"][best][None], 10000, axis=0)
    flip = np.random.default_rng(8).integers(0, 2, size=rows.shape).astype(np.uint8)
    flip[(rows & 0x7F) >= 0x7E] = 0
    d["k_idx"] = d["k_idx"].copy()
    d["k_idx"][20000:30000] = rows ^ flip
    run_case(dev, d, cfg.Lk, cfg.T, cfg.k, oracle_rows=(0,))


def test_prefill_topk_workspace_reuse(dev):
    cfg = synth.DecodeConfig("w", L=30000, T=24, k=512, plant_frac=0.01, seed=5)
    d = synth.decode_inputs(cfg, with_kv=False)
    qd, wd, kd = g(d["q_idx"], dev), g(d["w"], dev), g(d["k_idx"], dev)
    ws = binding.Workspace()
    a = binding.dsa_prefill_topk(qd, wd, kd, cfg.Lk, cfg.T, cfg.k, ws=ws).cpu().numpy()
    binding.dsa_prefill_topk(qd[:10], wd[:10], kd, 9000, 10, 2048, ws=ws)
    b = binding.dsa_prefill_topk(qd, wd, kd, cfg.Lk, cfg.T, cfg.k, ws=ws).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.timeout(900)
def test_prefill_topk_full_chunk(dev):
    cfg = synth.CONFIGS["dsa_prefill_1m_t8k"]
    T, Lk, k = cfg.T, cfg.Lk, cfg.k
    d = synth.decode_inputs(cfg, with_kv=False)
    print(f"\ndsa_prefill_1m_t8k fused top-k: Lk={Lk} T={T}", flush=True)
    qd, wd, kd = g(d["q_idx"], dev), g(d["w"], dev), g(d["k_idx"], dev)
    idx = binding.dsa_prefill_topk(qd, wd, kd, Lk, T, k)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    ws = binding.Workspace()
    for r0 in (0, 4096, T - 16):
        ref, _ = unfused(qd, wd, kd, Lk, T, k, r0, r0 + 16, ws)
        assert np.array_equal(idx_h[r0:r0 + 16], ref), f"rows {r0}.. differ from the unfused path"
    print("GPU done; checking rows against the oracle", flush=True)
    check_rows_oracle(d, Lk, T, k, idx_h, (0, T - 1))
