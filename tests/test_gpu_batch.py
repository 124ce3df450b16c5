"""GPU parity of the batched decode step (dsa_decode_batch) through the C ABI.

B ragged sequences share one index-key cache and one K/V cache; gaps between
them hold poison (random index keys, NaN K/V rows), so a read outside a
sequence shows up in its selection or output.  Per sequence, the selection
must equal bit for bit the top-k of the GPU's exact scores for that sequence
alone (dsa_index_scores on groups of at most 8 rows: the same arithmetic),
obey the top-k rule against the fp64 oracle at the 1e-4 near-tie band, and
the attention must match the oracle over that set.  Cases: serving (T = 1)
with lengths from 17 to 70,000, the 4-token verify, T = 12 and 16 (two scans
of token groups), empty and invalid sequence descriptors,
and the 64-sequence serving workload on a sample of sequences.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_long_context_index_amd import binding, synth
from test_gpu_parity import exact_scores, swap_report

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


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


def pack(seqs, rng, gap=37):
    """Concatenate the sequences' caches with poisoned gaps between them."""
    starts, rows = [], gap
    for s in seqs:
        starts.append(rows)
        rows += s["k_idx"].shape[0] + gap
    n_rows = rows
    k_idx = rng.integers(0, 0x7E, size=(n_rows, 128)).astype(np.uint8)      # poison: real-looking keys
    K = np.full((n_rows, 4, 192), BF16_NAN, np.uint16)
    V = np.full((n_rows, 4, 128), BF16_NAN, np.uint16)
    for s, st in zip(seqs, starts):
        n = s["k_idx"].shape[0]
        k_idx[st:st + n] = s["k_idx"]
        K[st:st + n] = s["k"]
        V[st:st + n] = s["v"]
    return k_idx, K, V, np.array(starts, np.int64), n_rows


def run_batch(dev, seqs, T, k, max_len=None, lens=None, starts=None, seed=0, sink=True):
    rng = np.random.default_rng(seed)
    k_idx, K, V, st, n_rows = pack(seqs, rng)
    lens = np.array([s["k_idx"].shape[0] for s in seqs], np.int32) if lens is None else np.asarray(lens, np.int32)
    st = st if starts is None else np.asarray(starts, np.int64)
    max_len = int(lens.max()) if max_len is None else max_len
    B = len(seqs)
    q_idx = np.stack([s["q_idx"] for s in seqs])
    w = np.stack([s["w"] for s in seqs])
    q = np.stack([s["q"] for s in seqs])
    idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    lse = torch.empty((B, T, 64), dtype=torch.float32, device=dev)
    out = binding.dsa_decode_batch(g(q_idx, dev), g(w, dev), g(k_idx, dev), g(q, dev), g(K, dev), g(V, dev),
                                   g(st, dev), g(lens, dev), max_len, k,
                                   g(seqs[0]["sink"], dev) if sink else None, float(seqs[0]["sm_scale"]),
                                   lse=lse, idx_out=idx)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy(), lse.cpu().numpy()


def check_seq(dev, s, T, k, o, idx, sink):
    Lk = s["k_idx"].shape[0]
    S = exact_scores(dev, g(s["q_idx"], dev), g(s["w"], dev), g(s["k_idx"], dev), Lk, T).cpu().numpy()
    assert np.array_equal(idx, oracle.topk(S.astype(np.float64), Lk, T, k)), "selection differs from the scores'"
    S_ref = oracle.index_scores(s["q_idx"], s["w"], s["k_idx"], Lk, T)
    idx_ref = oracle.topk(S_ref, Lk, T, k)
    msgs = []
    for t in range(T):
        n = Lk - T + t + 1
        ok, msg = oracle.topk_check(idx[t], idx_ref[t], S_ref[t, :n], k)
        assert ok, f"row {t}: {msg}"
        msgs.append(msg)
    swap_report(f"sequence of {Lk} keys, T={T}", msgs)
    o_ref, _ = oracle.sparse_attention(s["q"], s["k"], s["v"], idx, sink, float(s["sm_scale"]))
    ok, msg = oracle.attn_check(o, o_ref)
    assert ok, msg


@pytest.mark.parametrize("lens,T,k", [([300, 5000, 17, 40000, 2100], 1, 2048), ([70000, 9000, 131], 4, 2048),
                                      ([20000, 3000], 12, 2048), ([5000, 700, 12000], 16, 500),
                                      ([1, 2, 3, 4000], 1, 64)])
def test_decode_batch(dev, lens, T, k):
    lens = [max(n, T) for n in lens]
    seqs = synth.batch_inputs(lens, T, k, seed=sum(lens) + T)
    o, idx, _ = run_batch(dev, seqs, T, k, seed=len(lens))
    for b, s in enumerate(seqs):
        check_seq(dev, s, T, k, o[b], idx[b], seqs[0]["sink"])


def test_decode_batch_without_sink(dev):
    seqs = synth.batch_inputs([3000, 9000], 2, 256, seed=4)
    o, idx, _ = run_batch(dev, seqs, 2, 256, sink=False)
    for b, s in enumerate(seqs):
        check_seq(dev, s, 2, 256, o[b], idx[b], None)


def test_decode_batch_empty_and_invalid_sequences(dev):
    seqs = synth.batch_inputs([4000, 3000, 5000, 2000], 1, 512, seed=6)
    lens = [4000, 0, 5000, 2000]
    starts = None
    # sequence 1 is empty; sequence 3 claims more keys than max_len: both empty
    lens[3] = 6000
    o, idx, lse = run_batch(dev, seqs, 1, 512, max_len=5000, lens=lens, starts=starts)
    for b in (1, 3):
        assert np.all(idx[b] == -1)
        assert np.all(o[b] == 0)
        assert np.allclose(lse[b, 0], seqs[0]["sink"], atol=1e-6)     # only the sink in the denominator
    for b in (0, 2):
        check_seq(dev, seqs[b], 1, 512, o[b], idx[b], seqs[0]["sink"])


@pytest.mark.timeout(600)
def test_decode_batch_serving_workload(dev):
    # 64 sequences with lengths uniform in [256, 65536], one new token each
    lens = synth.batch_lengths(64, 256, 65536, seed=1005)
    seqs = synth.batch_inputs(lens, 1, 2048, seed=1005)
    o, idx, _ = run_batch(dev, seqs, 1, 2048, seed=5)
    for b in (0, int(np.argmax(lens)), int(np.argmin(lens)), 33):
        check_seq(dev, seqs[b], 1, 2048, o[b], idx[b], seqs[0]["sink"])


def test_decode_batch_many_sequences(dev):
    # more than 256 sequences: the scan gives each sequence a fixed share of
    # workgroups instead of dealing them by length
    lens = [int(n) for n in np.random.default_rng(9).integers(1, 3000, size=300)]
    seqs = synth.batch_inputs(lens, 1, 256, seed=9)
    o, idx, _ = run_batch(dev, seqs, 1, 256, seed=9)
    for b in (0, 1, 150, int(np.argmax(lens)), 299):
        check_seq(dev, seqs[b], 1, 256, o[b], idx[b], seqs[0]["sink"])


def test_decode_batch_256_sequences(dev):
    # the most sequences the length deal serves (256): at most 768 workgroups
    # are dealt, at least one per sequence
    lens = [int(n) for n in np.random.default_rng(11).integers(1, 20000, size=256)]
    seqs = synth.batch_inputs(lens, 1, 256, seed=11)
    o, idx, _ = run_batch(dev, seqs, 1, 256, seed=11)
    for b in (0, 7, 128, int(np.argmax(lens)), int(np.argmin(lens)), 255):
        check_seq(dev, seqs[b], 1, 256, o[b], idx[b], seqs[0]["sink"])
