"""The fused decode step captured in a HIP graph (as the benchmark and a
serving loop replay it) gives the eager result on every replay, with eager
work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

from sparse_long_context_index_amd import binding, synth
from test_gpu_parity import g

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda", 0)


def test_decode_step_graph_replays_match_eager(dev):
    cfg = synth.DecodeConfig("graph", L=70000, T=2, k=2048, plant_frac=0.01, seed=21)
    d = synth.decode_inputs(cfg)
    x = {n: g(d[n], dev) for n in ("q_idx", "w", "k_idx", "q", "k", "v", "sink")}
    Lk, T, k, sm = cfg.Lk, cfg.T, cfg.k, float(d["sm_scale"])
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_DECODE_STEP, Lk, T, k))
    out = torch.empty((T, 64, 128), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)

    def step():
        binding.dsa_decode_step(x["q_idx"], x["w"], x["k_idx"], x["q"], x["k"], x["v"], Lk, T, k, x["sink"], sm,
                                out=out, idx_out=idx, ws=ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_idx = out.clone(), idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = synth.decode_inputs(synth.DecodeConfig("o", L=3000, T=1, k=256, plant_frac=0.0, seed=3))
    for r in range(4):
        out.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {r}: out"
        assert torch.equal(idx, ref_idx), f"replay {r}: idx"
        # eager work on the same workspace between replays
        binding.dsa_decode_step(g(other["q_idx"], dev), g(other["w"], dev), g(other["k_idx"], dev), g(other["q"], dev),
                                g(other["k"], dev), g(other["v"], dev), 3001, 1, 256, g(other["sink"], dev),
                                float(other["sm_scale"]), ws=ws)
        torch.cuda.synchronize()
