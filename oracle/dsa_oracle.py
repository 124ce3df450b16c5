"""Plain fp64 CPU oracle for the DSA / SWA attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  The product path (the HIP
library and its Python binding) never touches it, and this module shares no
code with that path: it decodes the stored fp8 / bf16 bytes itself and computes
every step directly from its definition, slowly and in float64.

Citation keys used below (web pages about one model release):

* [NoFA]   "Naive-N0.5-Flash: no full-attention layers, and a runtime built by AI"
           (ai.thesatyajit.com): the property table, the section
           "What 'no full-attention layers' means", the section
           "Inside a DSA layer: the lightning indexer" with its Figure 1, and
           "How much of this did AI actually build?".
* [Master] "Naive-N0.5-Flash: the open-weight 309B MoE with no full-attention
           layers at all aims for 2,000 tokens/s per user" (ai-master.dev),
           section "Zero full-attention: what it really changes".

Readings taken where the pages are silent (each one is listed with its reason
in the design notes):

* fp8 is OCP E4M3FN with no scale factor; bf16 is the upper half of an IEEE
  binary32.
* query token t of T sits at position p_t = Lk - T + t and sees keys [0, p_t]
  (causal, including itself).
* index score S[t,s] = sum_h w[t,h] * max(q[t,h] . k[s], 0), no extra factor.
* top-k keeps the min(k, n_visible) keys ordered by (score descending, index
  ascending) and reports them in ascending index order, padded with -1.
* KV head of query head h is floor(h / (64 / Hkv)).
* the sink is one extra softmax logit per query head with no value vector,
  compared against the already-scaled logits (not multiplied by sm_scale).

Parity pins: every function here is checked by the ``-m "not gpu"`` tests
against closed forms, library special cases, invariants and brute force.
"""
from __future__ import annotations

import numpy as np

IDX_HEADS = 16
IDX_DIM = 128
Q_HEADS = 64
QK_DIM = 192
V_DIM = 128


# --------------------------------------------------------------------------
# O0: byte decoding.  [NoFA] property table: the indexer runs in fp8_e4m3;
# the main K/V are bf16 in the workloads we serve.
# --------------------------------------------------------------------------

def _build_e4m3_table() -> np.ndarray:
    """All 256 OCP E4M3FN codes as float64, from the format's definition:
    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (m/8 * 2^-6); codes 0x7F and 0xFF are NaN; there is no infinity,
    so exponent field 15 with mantissa < 7 is an ordinary normal number."""
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3_TABLE = _build_e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64: the bits are the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# O1: visibility.  [NoFA] Figure 1: the index sweep covers every visible key;
# SWA masks keys whose offset from the query reaches the window.
# --------------------------------------------------------------------------

def query_positions(Lk: int, T: int) -> np.ndarray:
    return np.arange(Lk - T, Lk, dtype=np.int64)


def swa_visible(p: int, s: int, window: int) -> bool:
    return 0 <= p - s < window


# --------------------------------------------------------------------------
# O2/O3: lightning-indexer scores.  [NoFA] "Inside a DSA layer": 16 fp8 query
# heads against one shared fp8 key head, ReLU of the dot product, combined by a
# learned per-head weight into one score per key.
# --------------------------------------------------------------------------

def index_logits(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """l[t,h,s] = sum_d q[t,h,d] * k[s,d] in float64.

    Exact: every e4m3 value is an integer multiple of 2^-9 of magnitude at most
    448, so each product is a multiple of 2^-18 below 2^36 units and a 128-term
    sum stays far inside float64's 53-bit significand, whatever the order."""
    q = decode_e4m3(q_idx)                       # [T,16,128]
    k = decode_e4m3(k_idx)                       # [Lk,128]
    return np.einsum("thd,sd->ths", q, k, optimize=True)


def index_scores(q_idx: np.ndarray, w: np.ndarray, k_idx: np.ndarray,
                 Lk: int, T: int) -> np.ndarray:
    """S[t,s] = sum_h w[t,h] * max(l[t,h,s], 0) for s <= p_t, -inf beyond."""
    assert q_idx.shape == (T, IDX_HEADS, IDX_DIM) and k_idx.shape[0] >= Lk
    out = np.full((T, Lk), -np.inf, dtype=np.float64)
    pos = query_positions(Lk, T)
    wf = np.asarray(w, dtype=np.float64)
    for t in range(T):
        n = int(pos[t]) + 1
        lg = index_logits(q_idx[t:t + 1], k_idx[:n])[0]          # [16, n]
        out[t, :n] = wf[t] @ np.maximum(lg, 0.0)
    return out


# --------------------------------------------------------------------------
# O4: top-k.  [NoFA] "What 'no full-attention layers' means": the DSA path
# keeps the first index_top_k entries of a descending argsort of the scores;
# "How much of this did AI actually build?": ties are stable (lower index
# first).
# --------------------------------------------------------------------------

def topk_row(scores_vis: np.ndarray, k: int) -> np.ndarray:
    """Indices of the top min(k, n) entries of a visible score prefix, ordered
    by (score desc, index asc), returned ascending and padded with -1 to k."""
    n = scores_vis.shape[0]
    s = np.arange(n, dtype=np.int64)
    order = np.lexsort((s, -np.asarray(scores_vis, dtype=np.float64)))
    take = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:take.size] = take
    return out


def topk(scores: np.ndarray, Lk: int, T: int, k: int) -> np.ndarray:
    pos = query_positions(Lk, T)
    return np.stack([topk_row(scores[t, :int(pos[t]) + 1], k) for t in range(T)])


# --------------------------------------------------------------------------
# O5: sparse GQA attention with sink.  [NoFA] "Inside a DSA layer": the main
# heads attend only to the selected keys (everything else is masked before the
# softmax); GQA with 4 KV heads on DSA layers and 8 on SWA layers; the sink is
# an extra softmax column.  [Master] "Zero full-attention": a sink bias on both
# attention types.
# --------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sink, sm_scale: float):
    """Softmax attention of one query head over an explicit key list.

    q [192] f64, K [n,192], V [n,128]; sink is a float or None.
    Returns (o [128], lse).  With m = max(max_j z_j, sink) and
    Z = sum_j e^(z_j - m) + e^(sink - m):  o = sum_j e^(z_j - m) V_j / Z,
    lse = m + ln Z.  An empty list gives o = 0, lse = sink (or -inf)."""
    n = K.shape[0]
    if n == 0:
        return np.zeros(V_DIM), (float(sink) if sink is not None else -np.inf)
    z = float(sm_scale) * (K @ q)
    m = z.max() if sink is None else max(z.max(), float(sink))
    e = np.exp(z - m)
    Z = e.sum() + (np.exp(float(sink) - m) if sink is not None else 0.0)
    return (e @ V) / Z, m + np.log(Z)


def sparse_attention(q_bits, k_bits, v_bits, idx, sink, sm_scale: float):
    """o[t,h] over the keys idx[t] (entries < 0 are empty slots).

    q_bits [T,64,192], k_bits [Lk,Hkv,192], v_bits [Lk,Hkv,128] bf16 bits;
    idx [T,k] int; sink [64] or None.  Returns out [T,64,128], lse [T,64]."""
    T = q_bits.shape[0]
    hkv = k_bits.shape[1]
    grp = Q_HEADS // hkv
    out = np.zeros((T, Q_HEADS, V_DIM))
    lse = np.zeros((T, Q_HEADS))
    for t in range(T):
        sel = np.asarray(idx[t], dtype=np.int64)
        sel = sel[sel >= 0]
        Kt = decode_bf16(k_bits[sel])                 # [n,Hkv,192]
        Vt = decode_bf16(v_bits[sel])                 # [n,Hkv,128]
        qt = decode_bf16(q_bits[t])                   # [64,192]
        for h in range(Q_HEADS):
            g = h // grp
            sg = None if sink is None else float(sink[h])
            out[t, h], lse[t, h] = attend(qt[h], Kt[:, g], Vt[:, g], sg, sm_scale)
    return out, lse


# --------------------------------------------------------------------------
# O6: sliding-window attention.  [NoFA] "What 'no full-attention layers'
# means": the SWA path keeps keys whose offset from the query is below the
# window; the window is 128 and includes the query itself.
# --------------------------------------------------------------------------

def swa_window(n: int, window: int) -> np.ndarray:
    """Positions a query at position n-1 sees in a sequence of n tokens."""
    p = n - 1
    return np.array([s for s in range(max(0, n - window), n) if swa_visible(p, s, window)],
                    dtype=np.int64)


def swa_attention(q_bits, k_win, v_win, seq_len, window: int, sink, sm_scale: float):
    """Single-token SWA decode for a ragged batch.

    q_bits [B,64,192]; k_win[b] / v_win[b] hold the LAST min(n_b, window) rows
    of sequence b's cache ([rows,8,*] bf16 bits).  Returns out [B,64,128],
    lse [B,64]."""
    B = q_bits.shape[0]
    out = np.zeros((B, Q_HEADS, V_DIM))
    lse = np.zeros((B, Q_HEADS))
    for b in range(B):
        n = int(seq_len[b])
        pos = swa_window(n, window)
        first = n - k_win[b].shape[0]           # position of k_win[b][0]
        rows = pos - first
        K = decode_bf16(k_win[b][rows])
        V = decode_bf16(v_win[b][rows])
        grp = Q_HEADS // K.shape[1]
        q = decode_bf16(q_bits[b])
        for h in range(Q_HEADS):
            sg = None if sink is None else float(sink[h])
            out[b, h], lse[b, h] = attend(q[h], K[:, h // grp], V[:, h // grp], sg, sm_scale)
    return out, lse


# --------------------------------------------------------------------------
# Composition: one DSA decode step (indexer -> top-k -> sparse attention),
# the order of [NoFA] Figure 1.
# --------------------------------------------------------------------------

def dsa_decode_step(inp: dict, k: int, sink=True):
    T = inp["q_idx"].shape[0]
    Lk = inp["k_idx"].shape[0]
    S = index_scores(inp["q_idx"], inp["w"], inp["k_idx"], Lk, T)
    idx = topk(S, Lk, T, k)
    out, lse = sparse_attention(inp["q"], inp["k"], inp["v"], idx,
                                inp["sink"] if sink else None, float(inp["sm_scale"]))
    return S, idx, out, lse


# --------------------------------------------------------------------------
# Index-selection recall ([NoFA] "How much of this did AI actually build?":
# the indexer's top-k was checked against a full-attention reference).  The
# share of each head's dense softmax mass, over every visible key and without
# the sink, that falls on the selected keys.
# --------------------------------------------------------------------------

def index_recall(q_bits, k_bits, idx, Lk: int, T: int, sm_scale: float):
    """recall [T,64] and the dense log-sum-exp lse_dense [T,64] (natural log)
    of the logits sm_scale * q . k over keys 0 .. p_t."""
    hkv = k_bits.shape[1]
    grp = Q_HEADS // hkv
    rec = np.zeros((T, Q_HEADS))
    lse = np.zeros((T, Q_HEADS))
    for t in range(T):
        n = Lk - T + t + 1
        Kt = decode_bf16(k_bits[:n])                  # [n,Hkv,192]
        qt = decode_bf16(q_bits[t])                   # [64,192]
        sel = np.asarray(idx[t], dtype=np.int64)
        sel = sel[(sel >= 0) & (sel < n)]
        for h in range(Q_HEADS):
            z = sm_scale * (Kt[:, h // grp] @ qt[h])
            m = z.max()
            e = np.exp(z - m)
            tot = e.sum()
            rec[t, h] = e[sel].sum() / tot
            lse[t, h] = m + np.log(tot)
    return rec, lse


def dsa_decode_batch(seqs: list, k: int, sink=True):
    """Decode step of several sequences: each is its own DSA decode step over
    its own keys (sharing a cache is storage, not arithmetic), so the batch is
    the list of per-sequence steps."""
    return [dsa_decode_step(s, k, sink) for s in seqs]


# --------------------------------------------------------------------------
# Acceptance helpers (tolerances from the arithmetic; used by the tests).
# --------------------------------------------------------------------------

def score_error_bound(q_idx: np.ndarray, w: np.ndarray, k_idx: np.ndarray,
                      Lk: int, T: int, rel: float = 2e-5) -> np.ndarray:
    """Per-score bound rel * sum_h |w_h| * sum_d |q_hd k_d| (+1e-30) on the
    error of a score computed in float32: exact fp8 products, float32 sums of
    the 128-term dots in any order, ReLU, float32 products with w and a
    float32 sum of the 16 heads.  The classical bound of an n-term float32
    sum in any order is (n-1) u sum |x_i| with u = 2^-24; the two sums chained
    give at most about (127 + 16) u sum_h |w_h| sum_d |q_hd k_d| = 8.5e-6 of
    it, so rel = 2e-5 holds with a factor-2 margin."""
    qa = np.abs(decode_e4m3(q_idx))
    ka = np.abs(decode_e4m3(k_idx[:Lk]))
    aw = np.abs(np.asarray(w, dtype=np.float64))
    out = np.zeros((T, Lk))
    for t in range(T):
        out[t] = aw[t] @ (qa[t] @ ka.T)
    return rel * out + 1e-30


def topk_check(gpu_idx_row: np.ndarray, ref_idx_row: np.ndarray,
               scores_vis: np.ndarray, k: int, rel_gap: float = 1e-4):
    """Top-k acceptance: the sets are equal except inside the near-tie band
    around the oracle's k-th score tau, |S_s - tau| <= rel_gap * |tau| (a
    floor of 1e-6 of the largest |score| keeps the band open when tau is 0).
    Returns (ok, message); the message starts with the number of swaps."""
    n = scores_vis.shape[0]
    g = np.asarray(gpu_idx_row, dtype=np.int64)
    r = np.asarray(ref_idx_row, dtype=np.int64)
    gs = g[g >= 0]
    rs = r[r >= 0]
    if gs.size != rs.size:
        return False, f"size {gs.size} != {rs.size}"
    if np.any(g[gs.size:] != -1):
        return False, "padding is not a -1 tail"
    if np.unique(gs).size != gs.size:
        return False, "duplicates"
    if gs.size and (gs.min() < 0 or gs.max() >= n):
        return False, "index out of visible range"
    if np.any(np.diff(gs) <= 0):
        return False, "not ascending"
    if gs.size == 0:
        return True, "empty"
    tau = scores_vis[rs].min()
    smax = np.abs(scores_vis).max()
    band = rel_gap * max(abs(tau), 1e-6 * smax)
    diff = np.setxor1d(gs, rs)
    bad = diff[np.abs(scores_vis[diff] - tau) > band]
    if bad.size:
        return False, f"{bad.size} disagreements outside the near-tie band"
    return True, f"{diff.size // 2} swaps inside the near-tie band"


def attn_check(o_gpu: np.ndarray, o_ref: np.ndarray, atol=2e-3, rtol=1e-2, rel_l2=1e-2):
    err = np.abs(o_gpu - o_ref)
    ok_el = bool(np.all(err <= atol + rtol * np.abs(o_ref)))
    denom = np.linalg.norm(o_ref)
    r = float(np.linalg.norm(o_gpu - o_ref) / denom) if denom > 0 else float(np.linalg.norm(o_gpu))
    return ok_el and r <= rel_l2, f"max_abs={err.max():.3e} rel_l2={r:.3e}"


# --------------------------------------------------------------------------
# Key-read accounting of the all-sparse stack.  [NoFA] "What 'no full-
# attention layers' means": an SWA layer reads at most the window, a DSA layer
# at most top-k keys, a dense layer every cached key.
# --------------------------------------------------------------------------

def backbone_keys_per_token(L: int, n_swa: int = 39, n_dsa: int = 9, window: int = 128,
                            topk_: int = 2048, dense: bool = False) -> int:
    per_dsa = L if dense else min(L, topk_)
    return n_swa * min(L, window) + n_dsa * per_dsa
