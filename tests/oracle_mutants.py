"""Planted mistakes in the oracle, for checking that its pins catch them.

Each entry replaces one oracle function with a copy that carries a plausible
slip (a dropped term, a wrong sign or index, a swapped operand, an
off-by-one).  ``tests/conftest.py`` applies the entry named by the
``BSATTN_ORACLE_MUTANT`` environment variable when pytest starts, so the
oracle pin tests then run against the mistaken oracle;
``tests/test_oracle_mutants.py`` asserts that each such run fails.  Nothing
here is used by the library, the bench or the normal test run.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention as oa
from oracle import heuristic as oh
from oracle import mask as om
from oracle import xattn as ox

BLOCK = 64


# ---- masks ----------------------------------------------------------------

def _topk_ties_high(scores, topk, dense_last_two_rows=False, force_diagonal=True):
    scores = np.asarray(scores)
    nb = scores.shape[-1]
    # slip: ties go to the higher column
    order = nb - 1 - np.argsort(-scores[..., ::-1], axis=-1, kind="stable")
    mask = np.zeros(scores.shape, dtype=np.uint8)
    np.put_along_axis(mask, order[..., :topk], 1, axis=-1)
    return om._finish(mask, dense_last_two_rows, force_diagonal)


def _threshold_ge(scores, threshold, dense_last_two_rows=False, force_diagonal=True):
    mask = (np.asarray(scores) >= np.float32(threshold)).astype(np.uint8)   # slip: >=
    return om._finish(mask, dense_last_two_rows, force_diagonal)


def _finish_dense_after_tril(mask, dense_last_two_rows, force_diagonal):
    nb = mask.shape[-1]
    mask = np.tril(mask)
    if dense_last_two_rows:   # slip: the dense rows set after the causal cut
        mask[..., max(0, nb - 2):, :] = 1
    if force_diagonal:
        d = np.arange(nb)
        mask[..., d, d] = 1
    return mask.astype(np.uint8)


def _finish_no_tril(mask, dense_last_two_rows, force_diagonal):
    nb = mask.shape[-1]
    if dense_last_two_rows:
        mask[..., max(0, nb - 2):, :] = 1
    if force_diagonal:        # slip: no causal cut
        d = np.arange(nb)
        mask[..., d, d] = 1
    return mask.astype(np.uint8)


def _indices_strict(mask, is_causal):
    mask = np.asarray(mask)
    B, H, nb, _ = mask.shape
    idx = np.full((B, H, nb, nb), -1, dtype=np.int32)
    cnt = np.zeros((B, H, nb), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                cols = np.flatnonzero(mask[b, h, i] != 0)
                if is_causal:
                    cols = cols[cols < i]          # slip: drops the diagonal
                idx[b, h, i, :cols.size] = cols
                cnt[b, h, i] = cols.size
    return idx, cnt


# ---- prefill --------------------------------------------------------------

def _prefill_rows(scale=None, strict=False, no_past=False, transposed=False, nan_empty=False):
    def f(q, k, v, block_mask, is_causal, rows=None):
        Sq, D = q.shape
        Sk = k.shape[0]
        past = 0 if no_past else Sk - Sq
        rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
        t = np.arange(Sk)
        kb = t // BLOCK
        s = (q[rows] @ k.T) / (scale(D) if scale else math.sqrt(D))
        if transposed:
            allowed = block_mask[kb][:, rows // BLOCK].T != 0   # slip: query and key block swapped
        else:
            allowed = block_mask[rows // BLOCK][:, kb] != 0
        if is_causal:
            lim = rows[:, None] + past
            allowed &= (t[None, :] < lim) if strict else (t[None, :] <= lim)
        if nan_empty:
            s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            return (p @ v) / p.sum(axis=-1, keepdims=True)
        return oa._softmax_rows(s, allowed, v)
    return f


# ---- decode ---------------------------------------------------------------

def _allowed_tokens(neg_ok=False, no_cut=False):
    def f(len_b, indices):
        nbb = -(-int(len_b) // BLOCK)
        toks = set()
        for i in indices:
            i = int(i)
            if (i < nbb) if neg_ok else (0 <= i < nbb):
                end = BLOCK * i + BLOCK if no_cut else min(BLOCK * i + BLOCK, int(len_b))
                toks.update(range(BLOCK * i, end))
        return np.array(sorted(toks), dtype=np.int64)
    return f


def _decode_head_modulo(q, k, v, cu_seqlens_k, block_indices):
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, Hq, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        start, end = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        for hq in range(Hq):
            kvh = hq % Hkv                       # slip: interleaved head mapping
            toks = oa.decode_allowed_tokens(end - start, block_indices[b, kvh])
            if toks.size:
                out[b, hq] = oa._attend_one(q[b, hq], k[start + toks, kvh], v[start + toks, kvh])
    return out


def _merge_exp(o_parts, lse2_parts):
    lse = np.asarray(lse2_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    mx = lse.max(axis=-1, keepdims=True)
    finite = np.isfinite(mx)
    mx = np.where(finite, mx, 0.0)
    w = np.exp(lse - mx)                           # slip: natural exponent on base-2 sums
    den = w.sum(axis=-1, keepdims=True)
    num = (w[..., None] * o).sum(axis=-2)
    den = np.where(den > 0, den, 1.0)
    return np.where(finite, num / den, 0.0)


def _paged_row_in_block(q, k_cache, v_cache, cache_seqlens, block_table, block_indices):
    B, Hq, D = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    G = Hq // Hkv
    r = page_size // BLOCK
    out = np.zeros((B, Hq, v_cache.shape[-1]), dtype=np.float64)
    for b in range(B):
        len_b = int(cache_seqlens[b])
        for hq in range(Hq):
            kvh = hq // G
            ok = [int(i) for i in block_indices[b, kvh]
                  if int(i) >= 0 and int(i) // r < block_table.shape[1]
                  and 0 <= int(block_table[b, int(i) // r]) < num_pages]
            toks = oa.decode_allowed_tokens(len_b, ok)
            if toks.size == 0:
                continue
            pages = block_table[b, toks // page_size].astype(np.int64)
            rows = toks % BLOCK                    # slip: row within the block, not the page
            out[b, hq] = oa._attend_one(q[b, hq], k_cache[pages, rows, kvh], v_cache[pages, rows, kvh])
    return out


# ---- estimator ------------------------------------------------------------

def _reshape_forward_both(q, k, stride):
    s = stride
    kr = np.concatenate([k[..., j::s, :] for j in range(s)], axis=-1)
    qr = np.concatenate([q[..., j::s, :] for j in range(s)], axis=-1)   # slip: not reversed
    return qr, kr


def _block_sums(no_stride=False, norm_mul=False, no_past=False):
    def f(q, k, stride, norm=1.0, causal=True):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        Sq, D = q.shape[-2], q.shape[-1]
        Sk = k.shape[-2]
        s = stride
        qr, kr = ox.stride_reshape(q, k, s)
        den = np.sqrt(D) * (1 if no_stride else s)
        den = den / norm if norm_mul else den * norm
        logits = (qr @ np.swapaxes(kr, -1, -2)) / den
        rq, rk = Sq // s, Sk // s
        if causal:
            past = 0 if no_past else (Sk - Sq) // s
            visible = np.arange(rk)[None, :] <= np.arange(rq)[:, None] + past
            logits = np.where(visible, logits, -np.inf)
        p = np.exp(logits - logits.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        b = BLOCK // s
        nbq, nbk = -(-Sq // BLOCK), -(-Sk // BLOCK)
        out = np.zeros(q.shape[:-2] + (nbq, nbk))
        for qi in range(nbq):
            for ki in range(nbk):
                out[..., qi, ki] = p[..., qi * b:(qi + 1) * b, ki * b:(ki + 1) * b].sum(axis=(-1, -2))
        return out
    return f


def _find_row(le=False, inclusive=False, keep_forced_weight=False):
    def f(x, threshold, sink, diag, causal_last):
        x = np.asarray(x, np.float32).astype(np.float64)
        n = x.shape[0]
        total = ox._sequential_sum(x)
        required = float(np.float32(threshold)) * total
        keep = np.zeros(n, bool)
        for c in (sink, diag):
            if c is not None and 0 <= c < n:
                keep[c] = True
        other = x if keep_forced_weight else np.where(keep, 0.0, x)
        order = np.argsort(-other, kind="stable")
        before = 0.0
        for c in order:
            upto = before + other[c] if inclusive else before
            if (upto <= required) if le else (upto < required):
                keep[c] = True
            before += other[c]
        if causal_last is not None:
            keep[causal_last + 1:] = False
        return keep.astype(np.uint8)
    return f


# ---- split heuristic ------------------------------------------------------

def _heuristic(fill=0.8, strict_fill=False, frac=0.85, largest=False):
    def f(total_mblocks, num_sms, num_n_blocks, num_m_blocks, size_one_kv_head,
          is_causal_or_local, max_splits):
        full = total_mblocks > fill * num_sms if strict_fill else total_mblocks >= fill * num_sms
        if full:
            if (size_one_kv_head > oh.L2_BYTES and num_m_blocks >= 2 * num_sms
                    and not is_causal_or_local):
                return min(math.ceil(size_one_kv_head / oh.L2_BYTES), max_splits)
            return 1
        if num_n_blocks <= 4:
            return 1
        cap = min(max_splits, num_sms, num_n_blocks)
        eff = [(total_mblocks * s / num_sms) / math.ceil(total_mblocks * s / num_sms)
               for s in range(1, cap + 1)]
        best = max(eff)
        ok = [s for s, e in enumerate(eff, start=1) if e >= frac * best]
        return ok[-1] if largest else ok[0]
    return f


# name -> (pin test files, run first to last; (module, attribute, replacement))
MUTANTS = {
    "mask_topk_ties_high": (["test_oracle_mask.py"], (om, "build_mask_topk", _topk_ties_high)),
    "mask_threshold_ge": (["test_oracle_mask.py"], (om, "build_mask_threshold", _threshold_ge)),
    "mask_dense_after_tril": (["test_oracle_mask.py"], (om, "_finish", _finish_dense_after_tril)),
    "mask_no_tril": (["test_oracle_mask.py"], (om, "_finish", _finish_no_tril)),
    "lists_drop_diagonal": (["test_oracle_mask.py"], (om, "mask_to_indices", _indices_strict)),
    "prefill_scale_1_over_d": (["test_oracle_attention.py"],
                               (oa, "prefill_head_rows", _prefill_rows(scale=lambda d: d))),
    "prefill_causal_strict": (["test_oracle_attention.py"],
                              (oa, "prefill_head_rows", _prefill_rows(strict=True))),
    "prefill_causal_no_past": (["test_oracle_prefill_chunk.py"],
                               (oa, "prefill_head_rows", _prefill_rows(no_past=True))),
    "prefill_mask_transposed": (["test_oracle_attention.py"],
                                (oa, "prefill_head_rows", _prefill_rows(transposed=True))),
    "prefill_empty_row_nan": (["test_oracle_attention.py", "test_oracle_prefill_chunk.py"],
                              (oa, "prefill_head_rows", _prefill_rows(nan_empty=True))),
    "decode_negative_index_wraps": (["test_oracle_attention.py", "test_oracle_decode_variants.py"],
                                    (oa, "decode_allowed_tokens", _allowed_tokens(neg_ok=True))),
    "decode_last_block_uncut": (["test_oracle_attention.py", "test_oracle_decode_variants.py"],
                                (oa, "decode_allowed_tokens", _allowed_tokens(no_cut=True))),
    "decode_head_modulo": (["test_oracle_attention.py", "test_oracle_decode_wide.py"],
                           (oa, "decode_gqa", _decode_head_modulo)),
    "merge_natural_exp": (["test_oracle_attention.py", "test_oracle_decode_variants.py"],
                          (oa, "merge_partials", _merge_exp)),
    "paged_row_in_block": (["test_oracle_decode_variants.py", "test_oracle_decode_wide.py"],
                           (oa, "decode_gqa_paged", _paged_row_in_block)),
    "xattn_query_not_reversed": (["test_oracle_xattn.py"], (ox, "stride_reshape", _reshape_forward_both)),
    "xattn_scale_without_stride": (["test_oracle_xattn.py"], (ox, "block_sums", _block_sums(no_stride=True))),
    "xattn_norm_multiplies": (["test_oracle_xattn.py"], (ox, "block_sums", _block_sums(norm_mul=True))),
    "xattn_causal_no_past": (["test_oracle_xattn.py"], (ox, "block_sums", _block_sums(no_past=True))),
    "select_keep_while_le": (["test_oracle_xattn.py"], (ox, "find_blocks_row", _find_row(le=True))),
    "select_inclusive_cumsum": (["test_oracle_xattn.py"], (ox, "find_blocks_row", _find_row(inclusive=True))),
    "select_forced_weight_ranked": (["test_oracle_xattn.py"],
                                    (ox, "find_blocks_row", _find_row(keep_forced_weight=True))),
    "splits_fill_strict": (["test_oracle_heuristic.py"],
                           (oh, "num_splits_heuristic", _heuristic(strict_fill=True))),
    "splits_fill_0_9": (["test_oracle_heuristic.py"], (oh, "num_splits_heuristic", _heuristic(fill=0.9))),
    "splits_frac_0_8": (["test_oracle_heuristic.py"], (oh, "num_splits_heuristic", _heuristic(frac=0.8))),
    "splits_largest": (["test_oracle_heuristic.py"], (oh, "num_splits_heuristic", _heuristic(largest=True))),
}


def apply(name: str) -> None:
    """Replace the oracle function the named entry targets (for this process)."""
    _, (module, attr, repl) = MUTANTS[name]
    assert hasattr(module, attr), (module.__name__, attr)
    setattr(module, attr, repl)
