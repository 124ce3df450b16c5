"""C-ABI checks that need no GPU: the library loads, exports every function
include/dsa.h declares, and rejects bad arguments before launching anything
(fake pointers below are never dereferenced because validation fails first)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_long_context_index_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

A = 0x10000        # 16-byte aligned fake device address
MIS = 0x10004      # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libdsa.so not built")
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for name in ("dsa_index_scores", "dsa_topk", "sparse_gqa_attn", "swa_attn", "dsa_decode_step",
                 "dsa_workspace_bytes", "dsa_workspace_init", "dsa_status_string", "dsa_version"):
        assert name in fns


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        assert hasattr(L, f)


def test_status_strings_and_version(L):
    for code, name in binding.STATUS.items():
        assert L.dsa_status_string(code).decode().startswith(name)
    assert b"gfx950" in L.dsa_version()


def test_workspace_bytes(L):
    f = L.dsa_workspace_bytes
    assert f(binding.OP_INDEX_SCORES, 100, 1, 1, 0) == 0
    assert f(binding.OP_TOPK, 100, 1, 0, 0) == 0            # k = 0 is invalid
    assert f(binding.OP_TOPK, 100, 1, 2049, 0) == 0         # k > 2048
    assert f(binding.OP_DECODE_STEP, 100, 9, 16, 0) == 0    # T > 8
    a = f(binding.OP_TOPK, 1 << 20, 1, 2048, 0)
    b = f(binding.OP_TOPK, 1 << 10, 1, 2048, 0)
    assert a >= b >= (1 << 20)
    d = f(binding.OP_DECODE_STEP, (1 << 20) + 1, 1, 2048, 0)
    assert d >= (1 << 20) + 4 * ((1 << 20) + 1)             # counters + scores
    assert f(binding.OP_SWA_ATTN, 0, 0, 0, 64) > 0
    assert f(binding.OP_SPARSE_ATTN, 100, 8192, 2048, 0) > 0


def test_index_scores_validation(L):
    s = L.dsa_index_scores
    assert s(None, A, A, 100, 1, A, 100, None) == 1
    assert s(A, A, A, 100, 0, A, 100, None) == 2             # T = 0
    assert s(A, A, A, 5, 6, A, 6, None) == 2                 # T > Lk
    assert s(A, A, A, 100, 1, A, 99, None) == 2              # ld < Lk
    assert s(A, A, A, 1 << 31, 1, A, 1 << 31, None) == 2     # Lk too large
    assert s(MIS, A, A, 100, 1, A, 100, None) == 4
    assert s(A, A, A, 100, 1, MIS, 100, None) == 4


def test_topk_validation(L):
    t = L.dsa_topk
    big = 1 << 30
    assert t(A, 100, 100, 1, 0, A, A, big, None) == 2        # k = 0
    assert t(A, 100, 100, 1, 2049, A, A, big, None) == 2     # k > 2048
    assert t(A, 100, 100, 1, 16, A, None, big, None) == 5    # no workspace
    assert t(A, 100, 100, 1, 16, A, A, 100, None) == 5       # workspace too small
    assert t(None, 100, 100, 1, 16, A, A, big, None) == 1
    assert t(A, 100, 100, 1, 16, MIS, A, big, None) == 4


def test_attention_validation(L):
    f = L.sparse_gqa_attn
    big = 1 << 30
    assert f(A, A, A, 100, None, 1, 16, None, 0.07, A, None, A, big, None) == 1
    assert f(A, A, A, 100, A, 1, 0, None, 0.07, A, None, A, big, None) == 2
    assert f(A, A, A, 100, A, 1, 16, None, float("nan"), A, None, A, big, None) == 2
    assert f(A, A, A, 100, A, 1, 16, MIS, 0.07, A, None, A, big, None) == 4
    assert f(A, A, A, 100, A, 1, 16, None, 0.07, A, None, A, 10, None) == 5
    g = L.swa_attn
    assert g(A, A, A, 1000, A, A, 4, 0, None, 0.07, A, None, A, big, None) == 2      # window 0
    assert g(A, A, A, 1000, A, A, 4, 4096, None, 0.07, A, None, A, big, None) == 2   # window > 2048
    assert g(A, A, A, 1000, None, A, 4, 128, None, 0.07, A, None, A, big, None) == 1
    assert g(A, A, A, 1000, A, A, 0, 128, None, 0.07, A, None, A, big, None) == 2


def test_decode_step_validation(L):
    f = L.dsa_decode_step
    big = 1 << 34
    args = [A, A, A, A, A, A, 100, 1, 16, None, 0.07, A, None, None, None, 0, A, big, None]
    bad = list(args)
    bad[7] = 9                                               # T > 8
    assert f(*bad) == 2
    bad = list(args)
    bad[14] = A
    bad[15] = 50                                             # scores_out with ld < Lk
    assert f(*bad) == 2
    bad = list(args)
    bad[17] = 1000                                           # workspace too small
    assert f(*bad) == 5
    bad = list(args)
    bad[0] = None
    assert f(*bad) == 1


def test_binding_refuses_cpu_tensors(L):
    import torch
    x = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(binding.DsaError):
        binding.dsa_index_scores(x, x, x, 1, 1, scores=torch.zeros(1, 1))


def test_cache_append_validation(L):
    f = L.dsa_cache_append
    ok = [A] * 4
    def call(idx_q=A, idx_k=A, g=None, b=None, eps=1e-6, q=A, k=A, v=A, Lk=100, T=1, ri=42, rm=64,
             base=1e7, qo=A, kc=A, qq=A, kk=A, vv=A):
        return f(idx_q, idx_k, g, b, eps, q, k, v, Lk, T, ri, rm, base, qo, kc, qq, kk, vv, None)
    assert call(idx_q=None) == 1
    assert call(vv=None) == 1
    assert call(k=MIS) == 4
    assert call(g=MIS) == 4
    assert call(T=0) == 2
    assert call(Lk=0) == 2
    assert call(T=8193, Lk=10000) == 2
    assert call(ri=43) == 2                 # odd rotary dims
    assert call(rm=194) == 2                # beyond the head
    assert call(ri=0) == 2
    assert call(base=0.0) == 2
    assert call(base=float("nan")) == 2
    assert call(eps=-1.0) == 2


def test_prefill_topk_validation(L):
    f = L.dsa_prefill_topk
    ws_need = L.dsa_workspace_bytes(binding.OP_PREFILL_TOPK, 100000, 64, 2048, 0)
    assert ws_need > 64 * 8192 * 8                      # the candidate slots alone
    assert L.dsa_workspace_bytes(binding.OP_PREFILL_TOPK, 100000, 64, 0, 0) == 0
    assert L.dsa_workspace_bytes(binding.OP_PREFILL_TOPK, 100000, 64, 2049, 0) == 0
    assert L.dsa_workspace_bytes(binding.OP_PREFILL_TOPK, 10, 64, 16, 0) == 0     # Lk < T
    # a workspace sized for larger sizes serves smaller ones
    assert L.dsa_workspace_bytes(binding.OP_PREFILL_TOPK, 50000, 32, 7, 0) <= ws_need

    def call(q=A, w=A, k=A, Lk=100000, T=64, kk=2048, idx=A, ws=A, nb=ws_need):
        return f(q, w, k, Lk, T, kk, idx, ws, nb, None)
    assert call(q=None) == 1
    assert call(idx=None) == 1
    assert call(idx=MIS) == 4
    assert call(k=MIS) == 4
    assert call(T=0) == 2
    assert call(Lk=10) == 2
    assert call(kk=0) == 2
    assert call(kk=2049) == 2
    assert call(ws=None) == 5
    assert call(nb=ws_need - 1) == 5
    assert call(ws=MIS) == 4


def test_decode_batch_validation(L):
    f = L.dsa_decode_batch
    need = L.dsa_workspace_bytes(binding.OP_DECODE_BATCH, 65536, 1, 2048, 64)
    assert need > 64 * 65536 * 4                          # the scores of the batch
    assert L.dsa_workspace_bytes(binding.OP_DECODE_BATCH, 65536, 17, 2048, 64) == 0   # T > 16
    assert L.dsa_workspace_bytes(binding.OP_DECODE_BATCH, 65536, 1, 2048, 0) == 0
    assert L.dsa_workspace_bytes(binding.OP_DECODE_BATCH, 30000, 1, 100, 8) <= need

    def call(qi=A, w=A, ki=A, q=A, kc=A, vc=A, n_rows=10 ** 6, ss=A, sl=A, B=64, T=1, max_len=65536, k=2048,
             sink=A, sm=0.07, out=A, lse=None, idx=None, ws=A, nb=need):
        return f(qi, w, ki, q, kc, vc, n_rows, ss, sl, B, T, max_len, k, sink, sm, out, lse, idx, ws, nb, None)
    assert call(ss=None) == 1
    assert call(out=None) == 1
    assert call(sl=MIS) == 4
    assert call(idx=MIS) == 4
    assert call(B=0) == 2
    assert call(T=17) == 2
    assert call(max_len=0) == 2
    assert call(k=0) == 2
    assert call(n_rows=0) == 2
    assert call(sm=float("inf")) == 2
    assert call(ws=None) == 5
    assert call(nb=need - 1) == 5


def test_index_recall_validation(L):
    f = L.dsa_index_recall
    need = L.dsa_workspace_bytes(binding.OP_INDEX_RECALL, 1 << 20, 1, 2048, 0)
    assert need > 0
    assert L.dsa_workspace_bytes(binding.OP_INDEX_RECALL, 10, 11, 2048, 0) == 0

    def call(q=A, kc=A, vc=A, Lk=1 << 20, idx=A, T=1, k=2048, sm=0.07, rec=A, lse=None, ws=A, nb=need):
        return f(q, kc, vc, Lk, idx, T, k, sm, rec, lse, ws, nb, None)
    assert call(idx=None) == 1
    assert call(rec=None) == 1
    assert call(q=None) == 1
    assert call(rec=MIS) == 4
    assert call(lse=MIS) == 4
    assert call(T=0) == 2
    assert call(k=2049) == 2
    assert call(Lk=0) == 2
    assert call(sm=float("nan")) == 2
    assert call(nb=need - 1) == 5
