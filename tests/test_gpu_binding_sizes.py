"""The binding refuses a buffer shorter than the bytes a call reads or writes
there, before anything is launched.

Each short tensor here is a view of the first bytes of a full-size
allocation, so a call that was not refused would still stay inside memory the
test owns.
"""
import numpy as np
import pytest
import torch

from sparse_long_context_index_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    return torch.device("cuda", 0)


def short(t):
    """t's first row dropped (same storage, so nothing past t is ever reachable)"""
    return t[: t.shape[0] - 1]


def test_append_refuses_short_caches(dev):
    T, Lk = 2, 64
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=dev)
    idx_q, idx_k, q, k, v = bf(T, 16, 128), bf(T, 128), bf(T, 64, 192), bf(T, 4, 192), bf(T, 4, 128)
    kic = torch.zeros((Lk, 128), dtype=torch.uint8, device=dev)
    kc, vc = bf(Lk, 4, 192), bf(Lk, 4, 128)
    for name, args in (("k_idx_cache", (short(kic), kc, vc)), ("k_cache", (kic, short(kc), vc)),
                       ("v_cache", (kic, kc, short(vc)))):
        with pytest.raises(binding.DsaError, match=name):
            binding.dsa_cache_append(idx_q, idx_k, q, k, v, Lk, T, *args)
    with pytest.raises(binding.DsaError, match="q"):
        binding.dsa_cache_append(short(idx_q), idx_k, q, k, v, Lk, T, kic, kc, vc)
    torch.cuda.synchronize()


def test_decode_step_refuses_short_inputs(dev):
    T, Lk, k = 1, 4096, 256
    q_idx = torch.zeros((T, 16, 128), dtype=torch.uint8, device=dev)
    w = torch.zeros((T, 16), dtype=torch.float32, device=dev)
    k_idx = torch.zeros((Lk, 128), dtype=torch.uint8, device=dev)
    q = torch.zeros((T, 64, 192), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((Lk, 4, 192), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((Lk, 4, 128), dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(64, dtype=torch.float32, device=dev)
    out = torch.empty((T, 64, 128), dtype=torch.bfloat16, device=dev)
    ws = binding.Workspace(binding.workspace_bytes(binding.OP_DECODE_STEP, Lk, T, k))
    for name, a in (("k_idx", dict(k_idx=short(k_idx))), ("k_cache", dict(k_cache=short(kc))),
                    ("v_cache", dict(v_cache=short(vc)))):
        args = dict(q_idx=q_idx, w=w, k_idx=k_idx, q=q, k_cache=kc, v_cache=vc)
        args.update(a)
        with pytest.raises(binding.DsaError, match=name):
            binding.dsa_decode_step(args["q_idx"], args["w"], args["k_idx"], args["q"], args["k_cache"],
                                    args["v_cache"], Lk, T, k, sink, 0.1, out=out, ws=ws)
    idx_out = torch.empty((T, k), dtype=torch.int32, device=dev)
    with pytest.raises(binding.DsaError, match="idx_out"):
        binding.dsa_decode_step(q_idx, w, k_idx, q, kc, vc, Lk, T, k, sink, 0.1, out=out,
                                idx_out=idx_out.view(-1)[: k - 1], ws=ws)
    torch.cuda.synchronize()


def test_topk_and_attention_refuse_short_buffers(dev):
    T, Lk, k = 2, 1000, 64
    scores = torch.zeros((T, Lk), dtype=torch.float32, device=dev)
    with pytest.raises(binding.DsaError, match="scores"):
        binding.dsa_topk(scores.view(-1)[: T * Lk - 1], Lk, T, k, ld=Lk)
    idx = torch.zeros((T, k), dtype=torch.int32, device=dev)
    q = torch.zeros((T, 64, 192), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((Lk, 4, 192), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((Lk, 4, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.DsaError, match="k_cache"):
        binding.sparse_gqa_attn(q, short(kc), vc, Lk, idx, None, 0.1)
    B = 3
    lens = torch.from_numpy(np.array([10, 20, 30], dtype=np.int32)).to(dev)
    starts = torch.from_numpy(np.array([0, 10, 30], dtype=np.int64)).to(dev)
    qs = torch.zeros((B, 64, 192), dtype=torch.bfloat16, device=dev)
    kc8 = torch.zeros((60, 8, 192), dtype=torch.bfloat16, device=dev)
    vc8 = torch.zeros((60, 8, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.DsaError, match="v_cache"):
        binding.swa_attn(qs, kc8, short(vc8), starts, lens, 128, None, 0.1)
    torch.cuda.synchronize()
