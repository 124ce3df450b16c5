"""Plain fp64 CPU oracle for the cache-append step that precedes the DSA scan.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module; the product path never does,
and this module shares no code with it.

What it computes, per new token at position p (the step before the index sweep
in "Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI",
section "Inside a DSA layer: the lightning indexer" and its Figure 1, panel B):

* the lightning indexer's single key head is layer-normalised, rotated by
  partial RoPE and rounded to fp8 e4m3, then appended to the index-key cache;
* its 16 query heads are rotated by partial RoPE and rounded to fp8 e4m3;
* the main attention's query heads and its KV heads' keys are rotated by
  partial RoPE and rounded to bf16; keys and values are appended to the K/V
  cache.

The same page, later in that section, gives the rotary fraction (a third of
each head, partial_rotary_factor 0.334) and the rope base of the sparse layers
(10,000,000); "How much of this did AI actually build?" reports that precision
issues in positional encoding were found, which is why angles are formed here
in float64 at the token's absolute position.

Readings taken where the pages are silent (each listed in the design notes):

* rotary dims R = int(head_dim * 0.334), i.e. 42 for the 128-dim index heads
  and 64 for the 192-dim attention heads; the first R dims rotate and the rest
  pass through;
* the rotation pairs dim i with dim i + R/2 (the half-split convention):
  x'_i = x_i cos(a_i) - x_{i+R/2} sin(a_i),
  x'_{i+R/2} = x_{i+R/2} cos(a_i) + x_i sin(a_i), a_i = p * base^(-2i/R);
* LayerNorm over the 128 index-key dims with caller-given gain and bias and
  eps = 1e-6; only the index key is normalised (the page names the key);
* inputs are the post-projection activations in bf16; rounding to fp8 is
  round-to-nearest-even after clamping to +-448, to bf16 round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

from .dsa_oracle import decode_bf16

ROTARY_FACTOR = 0.334
DSA_ROPE_BASE = 1.0e7
LN_EPS = 1e-6


def rotary_dims(head_dim: int, factor: float = ROTARY_FACTOR) -> int:
    """Rotated leading dims of a head ([NoFA] "Inside a DSA layer": a third)."""
    return int(head_dim * factor)


def rope_angles(pos, R: int, base: float) -> np.ndarray:
    """a[p, i] = p * base^(-2i/R) for i < R/2, in float64."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 1)
    i = np.arange(R // 2, dtype=np.float64)
    return pos * base ** (-2.0 * i / R)


def rope(x: np.ndarray, pos, R: int, base: float) -> np.ndarray:
    """Partial RoPE of x[..., D] at positions pos (one per leading row of x).

    x has shape [N, ..., D]; pos has N entries.  Dims >= R are unchanged."""
    x = np.asarray(x, dtype=np.float64)
    ang = rope_angles(pos, R, base)                       # [N, R/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (R // 2,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    h = R // 2
    y = x.copy()
    y[..., :h] = x[..., :h] * c - x[..., h:R] * s
    y[..., h:R] = x[..., h:R] * c + x[..., :h] * s
    return y


def layer_norm(x: np.ndarray, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * gamma + beta."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y


def to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float64 values to fp8 e4m3 codes: round to nearest, ties to even,
    after clamping to +-448, straight from the format (1 sign bit, 4 exponent
    bits with bias 7, 3 fraction bits; exponent field 0 is subnormal, steps
    of 2^-9).  One rounding from float64, so no double rounding."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), 448.0)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)          # 0..8; 8 is the smallest normal
    nrm = ~sub
    f, E = np.frexp(a[nrm])                                           # a = f 2^E, f in [0.5, 1)
    e = E - 1                                                         # a = (2 f) 2^e
    m = np.rint(a[nrm] / np.ldexp(1.0, e - 3)).astype(np.int64)      # in [8, 16]
    up = m == 16
    e = np.where(up, e + 1, e)
    m = np.where(up, 8, m)
    code[nrm] = ((e + 7) << 3) | (m - 8)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 bit patterns: round to nearest, ties to
    even, on the 8-significant-bit grid of each binade (one rounding)."""
    x = np.asarray(x, dtype=np.float64)
    f, E = np.frexp(x)                                                # |x| = |f| 2^E
    step_exp = np.maximum(E - 8, -133)                                # bf16 subnormal step 2^-133
    r = np.rint(np.ldexp(x, -step_exp))
    y = np.ldexp(r, step_exp).astype(np.float32)                      # exact: a bf16 value
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def cache_append(inp: dict, Lk: int, T: int, base: float = DSA_ROPE_BASE,
                 r_idx: int = None, r_main: int = None, eps: float = LN_EPS) -> dict:
    """Exact (float64, then one rounding) outputs of the append step.

    inp holds bf16 bit patterns: idx_q [T,16,128], idx_k [T,128], q [T,64,192],
    k [T,Hkv,192], v [T,Hkv,128]; and float32 ln_gamma, ln_beta [128].
    Token t sits at position Lk - T + t.  Returns the unrounded float64 values
    ("*_exact") and their roundings (fp8 codes / bf16 bits)."""
    pos = np.arange(Lk - T, Lk, dtype=np.int64)
    r_idx = rotary_dims(128) if r_idx is None else r_idx
    r_main = rotary_dims(192) if r_main is None else r_main
    iq = rope(decode_bf16(inp["idx_q"]), pos, r_idx, base)
    ik = rope(layer_norm(decode_bf16(inp["idx_k"]), inp.get("ln_gamma"), inp.get("ln_beta"), eps),
              pos, r_idx, base)
    q = rope(decode_bf16(inp["q"]), pos, r_main, base)
    k = rope(decode_bf16(inp["k"]), pos, r_main, base)
    v = decode_bf16(inp["v"]).astype(np.float64)
    return {
        "idx_q_exact": iq, "idx_k_exact": ik, "q_exact": q, "k_exact": k,
        "idx_q": to_e4m3(iq), "idx_k": to_e4m3(ik), "q": to_bf16(q), "k": to_bf16(k),
        "v": np.asarray(inp["v"], dtype=np.uint16).copy(),
    }
