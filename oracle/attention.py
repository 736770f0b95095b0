"""Attention oracle: block-sparse prefill and sparse GQA decode, float64.

Test infrastructure only (see ``oracle/__init__``).

Prefill follows the reference check of the TileLang block-sparse
Flash-Attention guide (§5): expand the block mask to token level (each mask
entry covers a BLOCK x BLOCK tile, cut to S x S), intersect with the causal
lower triangle, and run an ordinary dense softmax attention.  In symbols, for
query row r of head (b, h):

    allowed(r, t) = M[b, h, r // BLOCK, t // BLOCK] != 0
                    and (not causal or t <= r) and t < S
    s_t = (q_r . k_t) / sqrt(D)          over allowed t
    O_r = sum_t softmax(s)_t v_t,        O_r = 0 when no t is allowed.

The in-block causal rule (key t visible iff t <= r) is the guide's §4.5
reading of "0 below the diagonal, -inf above it"; the empty-row value 0 is
the reading for rows that hit no block (the guide relies on exp2(-inf) = 0
and never forms such a row in its test).  The online softmax of §4.6 is a
re-association of exactly this sum, so the oracle does not reproduce it.

Decode follows the same guide's §6–§6.2 (sparse GQA decode over variable
length KV): query head hq reads KV head hq // (Hq / Hkv); the keys it sees
are the union, over the selected block indices of its (batch, KV head), of
the tokens [BLOCK*i, min(BLOCK*i + BLOCK, len_b)).  Indices < 0 (padding)
or >= ceil(len_b / BLOCK) select nothing.  KV is packed by ``cu_seqlens_k``.
The split-KV partition and log-sum-exp merge of §6.1 are again only a
re-association; ``merge_partials`` states that merge on its own so tests can
pin it against the unsplit result.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

BLOCK = 64


def _softmax_rows(s: np.ndarray, allowed: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Dense masked softmax attention for a stack of rows (float64)."""
    s = np.where(allowed, s, -np.inf)
    any_allowed = allowed.any(axis=-1)
    m = np.where(any_allowed, s.max(axis=-1, initial=-np.inf), 0.0)
    p = np.exp(s - m[:, None])          # exp(-inf) = 0 on disallowed keys
    denom = p.sum(axis=-1)
    out = p @ v
    safe = np.where(any_allowed, denom, 1.0)
    out = out / safe[:, None]
    out[~any_allowed] = 0.0
    return out


def prefill_head_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_mask: np.ndarray,
                      is_causal: bool, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """One (batch, head): q, k, v float64 [S, D]; block_mask [nb, nb].

    Returns float64 [len(rows), D] (all S rows when ``rows`` is None)."""
    S, D = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    t = np.arange(S)
    kb = t // BLOCK
    s = (q[rows] @ k.T) / math.sqrt(D)
    allowed = block_mask[rows // BLOCK][:, kb] != 0
    if is_causal:
        allowed &= t[None, :] <= rows[:, None]
    return _softmax_rows(s, allowed, v)


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_mask: np.ndarray,
            is_causal: bool, row_chunk: int = 256) -> np.ndarray:
    """q, k, v float64 [B, H, S, D]; block_mask [B, H, nb, nb] -> float64 [B, H, S, D].

    Rows are independent, so they are evaluated a chunk at a time only to
    bound memory."""
    B, H, S, D = q.shape
    out = np.empty((B, H, S, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, S, row_chunk):
                rows = np.arange(r0, min(S, r0 + row_chunk))
                out[b, h, rows] = prefill_head_rows(q[b, h], k[b, h], v[b, h], block_mask[b, h],
                                                    is_causal, rows)
    return out


def decode_allowed_tokens(len_b: int, indices: Iterable[int]) -> np.ndarray:
    """Sorted token positions (within the sequence) selected by ``indices``."""
    nbb = -(-int(len_b) // BLOCK)
    toks = set()
    for i in indices:
        i = int(i)
        if 0 <= i < nbb:
            toks.update(range(BLOCK * i, min(BLOCK * i + BLOCK, int(len_b))))
    return np.array(sorted(toks), dtype=np.int64)


def decode_gqa(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_k: np.ndarray,
               block_indices: np.ndarray) -> np.ndarray:
    """q float64 [B, Hq, D]; k, v float64 [total_k, Hkv, D]; cu_seqlens_k [B+1];
    block_indices [B, Hkv, max_sel] -> float64 [B, Hq, D]."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        start, end = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        for hq in range(Hq):
            kvh = hq // G
            toks = decode_allowed_tokens(end - start, block_indices[b, kvh])
            if toks.size == 0:
                continue
            kk = k[start + toks, kvh]            # [n, D]
            vv = v[start + toks, kvh]
            s = (kk @ q[b, hq]) / math.sqrt(D)
            p = np.exp(s - s.max())
            out[b, hq] = (p @ vv) / p.sum()
    return out


def merge_partials(o_parts: np.ndarray, lse2_parts: np.ndarray) -> np.ndarray:
    """Log-sum-exp merge of split results (guide §6.1, merge stage).

    o_parts [..., ns, D] are per-split normalised outputs, lse2_parts [..., ns]
    their base-2 log-sum-exp (-inf for a split that saw no key).  The result
    is sum_s w_s o_s / sum_s w_s with w_s = 2^(lse_s - max_s lse_s); it is 0
    when every split is empty."""
    lse = np.asarray(lse2_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    mx = lse.max(axis=-1, keepdims=True)
    finite = np.isfinite(mx)
    mx = np.where(finite, mx, 0.0)
    w = np.exp2(lse - mx)
    den = w.sum(axis=-1, keepdims=True)
    num = (w[..., None] * o).sum(axis=-2)
    den = np.where(den > 0, den, 1.0)
    return np.where(finite, num / den, 0.0)
