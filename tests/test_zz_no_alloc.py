"""GPU check of the no-allocation decode step (dsa_decode_step_noalloc) through
the C ABI: on the library's static per-GPU scratch it must give exactly the
bits of dsa_decode_step on a caller workspace -- on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents),
on the list path and on the histogram path (T > 4) -- and refuse a request
larger than the scratch before enqueuing anything.
"""
import numpy as np
import pytest
import torch

from sparse_long_context_index_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda", 0)


def inputs(dev, L, T, k, seed):
    cfg = synth.DecodeConfig("na", L=L, T=T, k=k, plant_frac=0.01, seed=seed)
    d = synth.decode_inputs(cfg)
    x = {}
    for n in ("q_idx", "w", "k_idx", "q", "k", "v", "sink"):
        a = np.ascontiguousarray(d[n])
        x[n] = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    return cfg, x, float(d["sm_scale"])


def outputs(dev, cfg, with_scores):
    T, k, Lk = cfg.T, cfg.k, cfg.Lk
    return (torch.full((T, 64, 128), 7, dtype=torch.int16, device=dev).view(torch.bfloat16),
            torch.full((T, 64), 7.0, dtype=torch.float32, device=dev),
            torch.full((T, k), 7, dtype=torch.int32, device=dev),
            torch.full((T, Lk), 7.0, dtype=torch.float32, device=dev) if with_scores else None)


def same(a, b):
    return a is None and b is None or torch.equal(a.view(torch.int32 if a.dtype == torch.float32 else a.dtype),
                                                  b.view(torch.int32 if b.dtype == torch.float32 else b.dtype))


@pytest.mark.parametrize("first,second", [((300000, 1, 2048, True), (20000, 1, 2048, False)),
                                          ((150000, 4, 2048, False), (9000, 2, 512, True)),
                                          ((60000, 6, 1000, True), (3000, 5, 2048, False))])
def test_noalloc_matches_the_workspace_call_twice(dev, first, second):
    for i, (L, T, k, with_scores) in enumerate((first, second)):
        cfg, x, sm = inputs(dev, L, T, k, seed=L + T + i)
        print(f"\ncall {i}: Lk={cfg.Lk} T={T} k={k} scores={with_scores}", flush=True)
        o1, l1, i1, s1 = outputs(dev, cfg, with_scores)
        binding.dsa_decode_step(x["q_idx"], x["w"], x["k_idx"], x["q"], x["k"], x["v"], cfg.Lk, T, k, x["sink"],
                                sm, out=o1, lse=l1, idx_out=i1, scores_out=s1)
        o2, l2, i2, s2 = outputs(dev, cfg, with_scores)
        binding.dsa_decode_step_noalloc(x["q_idx"], x["w"], x["k_idx"], x["q"], x["k"], x["v"], cfg.Lk, T, k,
                                        x["sink"], sm, out=o2, lse=l2, idx_out=i2, scores_out=s2)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2), "index sets differ"
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs"
        assert same(s1, s2), "scores differ"


def test_noalloc_refuses_requests_beyond_the_scratch(dev):
    # T = 8 over 2M keys needs ~100 MB of scratch: refused before any launch
    # (the inputs are never read, so small tensors stand in)
    small = torch.zeros(4096, dtype=torch.uint8, device=dev)
    lib = binding.load()
    p = lambda t: t.data_ptr()
    out = torch.zeros((8, 64, 128), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.dsa_decode_step_noalloc(p(small), p(small), p(small), p(small), p(small), p(small), 2_000_000, 8, 2048,
                                     None, 0.07, p(out), None, None, None, 0, st)
    assert binding.STATUS[rc] == "DSA_ERR_SCRATCH"
    assert lib.dsa_status_string(rc).startswith(b"DSA_ERR_SCRATCH")
    assert torch.count_nonzero(out.view(torch.int16)).item() == 0
