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

The in-block causal rule (key t visible iff t <= r) reads the guide's §4.5
in-block mask, which adds zero on and below the diagonal and minus infinity
above it; the empty-row value 0 is
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

Two decode variants of the same guide change only which tokens a head sees:
the mask form (§6, ``block_mask [B, Hkv, num_blocks]`` instead of indices)
and the paged KV cache (§7, K/V in fixed-size physical pages reached through
a per-sequence block table).
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
    """One (batch, head): q float64 [Sq, D]; k, v float64 [Sk, D] with Sk >= Sq;
    block_mask [ceil(Sq/64), ceil(Sk/64)].

    With Sk > Sq the queries are the last Sq positions of an Sk-token context
    (past = Sk - Sq, as the TileLang FlashAttention guide's BHSD example
    aligns the causal mask with ``q_idx = row + past_len``, and the
    block-sparse guide's §8 Triton reference with PAST_LEN): query row r sees
    key t when its block is selected, t < Sk, and, if causal, t <= r + past.

    Returns float64 [len(rows), D] (all Sq rows when ``rows`` is None)."""
    Sq, D = q.shape
    Sk = k.shape[0]
    past = Sk - Sq
    assert past >= 0
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    t = np.arange(Sk)
    kb = t // BLOCK
    s = (q[rows] @ k.T) / math.sqrt(D)
    allowed = block_mask[rows // BLOCK][:, kb] != 0
    if is_causal:
        allowed &= t[None, :] <= rows[:, None] + past
    return _softmax_rows(s, allowed, v)


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_mask: np.ndarray,
            is_causal: bool, row_chunk: int = 256) -> np.ndarray:
    """q float64 [B, H, Sq, D]; k, v float64 [B, H, Sk, D] (Sk >= Sq, usually
    equal); block_mask [B, H, ceil(Sq/64), ceil(Sk/64)] -> float64 [B, H, Sq, D].

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
    """q float64 [B, Hq, D]; k float64 [total_k, Hkv, D]; v float64
    [total_k, Hkv, Dv]; cu_seqlens_k [B+1]; block_indices [B, Hkv, max_sel]
    -> float64 [B, Hq, Dv].  The value head dim Dv may differ from the key
    head dim D (the guide's decode takes dim and dim_v, §9.2; the scores
    scale by D^-1/2)."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((B, Hq, v.shape[-1]), dtype=np.float64)
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


def _attend_one(qv: np.ndarray, kk: np.ndarray, vv: np.ndarray) -> np.ndarray:
    """softmax(kk . qv / sqrt(D)) vv for one query vector (float64)."""
    s = (kk @ qv) / math.sqrt(qv.shape[-1])
    p = np.exp(s - s.max())
    return (p @ vv) / p.sum()


def decode_gqa_mask(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_k: np.ndarray,
                    block_mask: np.ndarray) -> np.ndarray:
    """Mask-form sparse GQA decode (same guide, §6: the variant whose loop
    tests ``block_mask[b, kvh, j]`` where the index form tests
    ``block_indices >= 0``).  Block j of sequence b is selected for KV head
    kvh when block_mask[b, kvh, j] != 0 and j < ceil(len_b / 64); everything
    else is as in ``decode_gqa``.

    q float64 [B, Hq, D]; k float64 [total_k, Hkv, D]; v float64
    [total_k, Hkv, Dv]; cu_seqlens_k [B+1]; block_mask [B, Hkv, num_blocks]
    (nonzero = selected) -> float64 [B, Hq, Dv]."""
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((B, Hq, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        start, end = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        for hq in range(Hq):
            kvh = hq // G
            sel = [j for j in range(block_mask.shape[2]) if block_mask[b, kvh, j] != 0]
            toks = decode_allowed_tokens(end - start, sel)
            if toks.size:
                out[b, hq] = _attend_one(q[b, hq], k[start + toks, kvh], v[start + toks, kvh])
    return out


def decode_gqa_paged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     cache_seqlens: np.ndarray, block_table: np.ndarray,
                     block_indices: np.ndarray) -> np.ndarray:
    """Paged-KV sparse GQA decode (same guide, §7).

    k_cache float64 [num_pages, page_size, Hkv, D] and v_cache float64
    [num_pages, page_size, Hkv, Dv] with page_size a multiple of 64; block_table [B, max_blocks_per_seq] maps a sequence's
    logical page to a physical page; cache_seqlens [B] are the lengths.
    Logical 64-token block i of sequence b is rows (i % r) * 64 .. +63 of
    physical page block_table[b, i // r], r = page_size // 64, so token t
    sits at row t % page_size of page block_table[b, t // page_size].  An
    index selects nothing when it is < 0, >= ceil(len_b / 64), or its table
    entry is missing or outside [0, num_pages) (the memory-safe reading).
    Everything else is as in ``decode_gqa``.  -> float64 [B, Hq, Dv]."""
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    assert Hq % Hkv == 0 and page_size % BLOCK == 0
    G = Hq // Hkv
    r = page_size // BLOCK
    out = np.zeros((B, Hq, v_cache.shape[-1]), dtype=np.float64)
    for b in range(B):
        len_b = int(cache_seqlens[b])
        for hq in range(Hq):
            kvh = hq // G
            ok = []
            for i in block_indices[b, kvh]:
                i = int(i)
                if i < 0 or i // r >= block_table.shape[1]:
                    continue
                if 0 <= int(block_table[b, i // r]) < num_pages:
                    ok.append(i)
            toks = decode_allowed_tokens(len_b, ok)
            if toks.size == 0:
                continue
            pages = block_table[b, toks // page_size].astype(np.int64)
            rows = toks % page_size
            out[b, hq] = _attend_one(q[b, hq], k_cache[pages, rows, kvh], v_cache[pages, rows, kvh])
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
