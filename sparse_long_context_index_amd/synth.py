"""Seeded synthetic inputs for the DSA / SWA decode and prefill workloads.

This module is shared by the tests, the benchmark and the smoke check; it holds
none of the method's arithmetic (no index scores, no selection, no attention).
It only draws random numbers with numpy's PCG64 and encodes them into the byte
formats the kernels consume:

* fp8 OCP E4M3FN bytes (``torch.float8_e4m3fn`` cast, round-to-nearest-even,
  after clamping to +-448 because the cast turns out-of-range values into NaN);
* bf16 bit patterns (``torch.bfloat16`` cast, round-to-nearest-even).

Shapes follow the model constants read from the released config by
"Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI"
(property table): 16 index heads of dim 128 against one fp8_e4m3 index-key
head, 64 query heads with qk dim 192 and v dim 128, 4 KV heads on DSA layers
and 8 on SWA layers, top-2,048 selection, a 128-token window.

Workload recipe (one ``SeedSequence(seed).spawn`` child per tensor):

* index queries ``q_idx`` and index keys ``k_idx``: N(0,1) -> e4m3;
* per-head index weights ``w``: N(0,1) float32 (may be negative);
* attention ``Q``, ``K``, ``V``: N(0,1) -> bf16; the softmax scale 1/sqrt(192)
  is applied by the kernel, so logits are ~N(0,1);
* per-head sink logits: N(0,1) float32;
* planted keys: a fraction of the history positions (chosen without
  replacement) each get a random query token t and are rewritten as
  e4m3(z + gamma * u_t), where z is the key's own draw, u_t the unit vector of
  sum_h max(w[t,h], 0) * q[t,h] (sum_h q[t,h] if no weight is positive), and
  gamma = 8.  This makes the top-k non-trivial (planted keys score high).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

IDX_HEADS = 16
IDX_DIM = 128
Q_HEADS = 64
QK_DIM = 192
V_DIM = 128
DSA_KV_HEADS = 4
SWA_KV_HEADS = 8
TOPK = 2048
SWA_WINDOW = 128
PLANT_GAMMA = 8.0

# tensor -> spawn-child slot; fixed so that adding a tensor never reshuffles
# the streams of the others.
_SLOTS = {"q_idx": 0, "w": 1, "k_idx": 2, "q": 3, "k": 4, "v": 5, "sink": 6,
          "plant_pos": 7, "plant_tok": 8, "seq_len": 9,
          "ap_idx_q": 10, "ap_idx_k": 11, "ap_q": 12, "ap_k": 13, "ap_v": 14,
          "ln_gamma": 15, "ln_beta": 16, "batch_len": 17}

_CHUNK = 1 << 22  # elements per generation/encoding chunk


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """A DSA workload: T query tokens appended to a history of L tokens."""
    name: str
    L: int
    T: int
    k: int = TOPK
    plant_frac: float = 0.01
    seed: int = 0

    @property
    def Lk(self) -> int:
        # keys visible to the last query token: the history plus the T new tokens
        return self.L + self.T


@dataclasses.dataclass(frozen=True)
class SwaConfig:
    """A batch of single-token SWA decodes over ragged histories."""
    name: str
    B: int
    len_lo: int
    len_hi: int
    window: int = SWA_WINDOW
    seed: int = 0


CONFIGS = {
    "dsa_decode_8k": DecodeConfig("dsa_decode_8k", L=8192, T=1, plant_frac=0.01, seed=1000),
    "dsa_verify_128k_t4": DecodeConfig("dsa_verify_128k_t4", L=131072, T=4, plant_frac=0.005, seed=1001),
    "dsa_decode_1m": DecodeConfig("dsa_decode_1m", L=1048576, T=1, plant_frac=0.01, seed=1002),
    "swa_decode_b64": SwaConfig("swa_decode_b64", B=64, len_lo=256, len_hi=65536, seed=1003),
    "dsa_prefill_1m_t8k": DecodeConfig("dsa_prefill_1m_t8k", L=1048576, T=8192, plant_frac=0.01, seed=1004),
}


def _rng(seed: int, name: str) -> np.random.Generator:
    child = np.random.SeedSequence(seed).spawn(len(_SLOTS))[_SLOTS[name]]
    return np.random.Generator(np.random.PCG64(child))


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3FN bytes (RNE), clamped to +-448 first."""
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(flat.size, dtype=np.uint8)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        t = torch.from_numpy(flat[s:e]).clamp(-448.0, 448.0)
        out[s:e] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(x.shape)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (RNE) as uint16."""
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        t = torch.from_numpy(flat[s:e]).to(torch.bfloat16)
        out[s:e] = t.view(torch.int16).numpy().view(np.uint16)
    return out.reshape(x.shape)


def _e4m3_as_f32(codes: np.ndarray) -> np.ndarray:
    # generator-side decode (torch), used only to aim the planted keys
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def index_inputs(L: int, T: int, seed: int, plant_frac: float = 0.0,
                 plant_gamma: float = PLANT_GAMMA) -> Dict[str, np.ndarray]:
    """Indexer inputs for T query tokens over Lk = L + T keys.

    Returns q_idx [T,16,128] u8, w [T,16] f32, k_idx [Lk,128] u8 and the planted
    positions/tokens (int64 arrays, possibly empty).
    """
    Lk = L + T
    q_idx = encode_e4m3(normal_f32(_rng(seed, "q_idx"), (T, IDX_HEADS, IDX_DIM)))
    w = normal_f32(_rng(seed, "w"), (T, IDX_HEADS))
    z = normal_f32(_rng(seed, "k_idx"), (Lk, IDX_DIM))
    n_plant = int(round(plant_frac * L))
    if n_plant > 0:
        pos = _rng(seed, "plant_pos").choice(L, size=n_plant, replace=False)
        pos.sort()
        tok = _rng(seed, "plant_tok").integers(0, T, size=n_plant)
        qf = _e4m3_as_f32(q_idx).astype(np.float64)  # [T,16,128]
        wp = np.maximum(w.astype(np.float64), 0.0)
        d = np.einsum("th,thd->td", wp, qf)
        for t in range(T):
            if not np.any(wp[t] > 0):
                d[t] = qf[t].sum(axis=0)
        nrm = np.linalg.norm(d, axis=1, keepdims=True)
        nrm[nrm == 0] = 1.0
        u = (d / nrm).astype(np.float32)
        z[pos] += np.float32(plant_gamma) * u[tok]
    else:
        pos = np.zeros(0, dtype=np.int64)
        tok = np.zeros(0, dtype=np.int64)
    k_idx = encode_e4m3(z)
    del z
    return {"q_idx": q_idx, "w": w, "k_idx": k_idx,
            "plant_pos": pos.astype(np.int64), "plant_tok": tok.astype(np.int64)}


def attention_inputs(Lk: int, T: int, seed: int, n_kv_heads: int = DSA_KV_HEADS,
                     with_kv: bool = True) -> Dict[str, np.ndarray]:
    """Main-attention inputs: Q [T,64,192], K [Lk,Hkv,192], V [Lk,Hkv,128] (bf16
    bits as uint16) and sink [64] f32."""
    out = {
        "q": encode_bf16(normal_f32(_rng(seed, "q"), (T, Q_HEADS, QK_DIM))),
        "sink": normal_f32(_rng(seed, "sink"), (Q_HEADS,)),
    }
    if with_kv:
        out["k"] = encode_bf16(normal_f32(_rng(seed, "k"), (Lk, n_kv_heads, QK_DIM)))
        out["v"] = encode_bf16(normal_f32(_rng(seed, "v"), (Lk, n_kv_heads, V_DIM)))
    return out


def decode_inputs(cfg: DecodeConfig, with_kv: bool = True) -> Dict[str, np.ndarray]:
    d = index_inputs(cfg.L, cfg.T, cfg.seed, cfg.plant_frac)
    d.update(attention_inputs(cfg.Lk, cfg.T, cfg.seed, DSA_KV_HEADS, with_kv))
    d["sm_scale"] = np.float32(1.0 / math.sqrt(QK_DIM))
    return d


def swa_inputs(cfg: SwaConfig) -> Dict[str, np.ndarray]:
    """Ragged SWA batch.  Only each sequence's last ``window`` rows are drawn;
    the caller lays them into a full-length cache (the rest is poison).

    Returns seq_len [B] i32, seq_start [B] i64 (prefix sums of seq_len), q
    [B,64,192] u16, k_win / v_win lists of [min(n,window),8,*] u16, sink [64].
    """
    rng_len = _rng(cfg.seed, "seq_len")
    seq_len = rng_len.integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.B).astype(np.int32)
    seq_start = np.zeros(cfg.B, dtype=np.int64)
    seq_start[1:] = np.cumsum(seq_len.astype(np.int64))[:-1]
    nw = np.minimum(seq_len, cfg.window).astype(np.int64)
    tot = int(nw.sum())
    kk = encode_bf16(normal_f32(_rng(cfg.seed, "k"), (tot, SWA_KV_HEADS, QK_DIM)))
    vv = encode_bf16(normal_f32(_rng(cfg.seed, "v"), (tot, SWA_KV_HEADS, V_DIM)))
    offs = np.concatenate([[0], np.cumsum(nw)])
    return {
        "seq_len": seq_len, "seq_start": seq_start,
        "q": encode_bf16(normal_f32(_rng(cfg.seed, "q"), (cfg.B, Q_HEADS, QK_DIM))),
        "k_win": [kk[offs[b]:offs[b + 1]] for b in range(cfg.B)],
        "v_win": [vv[offs[b]:offs[b + 1]] for b in range(cfg.B)],
        "sink": normal_f32(_rng(cfg.seed, "sink"), (Q_HEADS,)),
        "sm_scale": np.float32(1.0 / math.sqrt(QK_DIM)),
    }


def batch_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded ragged key counts (history plus new tokens) of a decode batch,
    uniform in [lo, hi]."""
    return _rng(seed, "batch_len").integers(lo, hi + 1, size=B).astype(np.int64)


def batch_inputs(lengths, T: int, k: int, seed: int, plant_frac: float = 0.01) -> list:
    """Per-sequence decode inputs of a batch: sequence b has lengths[b] keys
    (its history and its T new tokens), drawn like decode_inputs."""
    return [decode_inputs(DecodeConfig(f"b{b}", L=int(n) - T, T=T, k=k, plant_frac=plant_frac,
                                       seed=seed * 1009 + b))
            for b, n in enumerate(lengths)]


def sample_rows(T: int, n: int = 64, seed: int = 4) -> np.ndarray:
    """Seeded row sample for checking a long prefill chunk: the first and last
    row plus n-2 distinct others, ascending."""
    if T <= n:
        return np.arange(T, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid])).astype(np.int64)


BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)


def append_inputs(T: int, seed: int, n_kv_heads: int = DSA_KV_HEADS) -> Dict[str, np.ndarray]:
    """Post-projection activations of T new tokens for the cache-append step.

    idx_q [T,16,128], idx_k [T,128], q [T,64,192], k [T,Hkv,192], v [T,Hkv,128]
    as bf16 bit patterns of N(0,1) draws; ln_gamma = 1 + 0.1 N(0,1) and
    ln_beta = 0.1 N(0,1) float32 [128] stand in for the index key's LayerNorm
    gain and bias."""
    return {
        "idx_q": encode_bf16(normal_f32(_rng(seed, "ap_idx_q"), (T, IDX_HEADS, IDX_DIM))),
        "idx_k": encode_bf16(normal_f32(_rng(seed, "ap_idx_k"), (T, IDX_DIM))),
        "q": encode_bf16(normal_f32(_rng(seed, "ap_q"), (T, Q_HEADS, QK_DIM))),
        "k": encode_bf16(normal_f32(_rng(seed, "ap_k"), (T, n_kv_heads, QK_DIM))),
        "v": encode_bf16(normal_f32(_rng(seed, "ap_v"), (T, n_kv_heads, V_DIM))),
        "ln_gamma": (1.0 + 0.1 * normal_f32(_rng(seed, "ln_gamma"), (IDX_DIM,))).astype(np.float32),
        "ln_beta": (0.1 * normal_f32(_rng(seed, "ln_beta"), (IDX_DIM,))).astype(np.float32),
    }
