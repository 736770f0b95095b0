"""Block-mask oracle: top-k and threshold builders, and row compaction.

Test infrastructure only (see ``oracle/__init__``).

Readings of the pages used here:

* top-k (TileLang block-sparse Flash-Attention guide, §3.1): each query-block
  row keeps the ``topk`` key blocks with the highest scores over the WHOLE
  row; ties, which the pages leave open, go to the lower column index.
* threshold (same guide, §3.2): a block is kept when its score is strictly
  greater than the threshold (the comparison operator was lost in the text;
  the prose keeps scores that exceed the threshold).
* optional dense last two block rows come BEFORE the causal tril (the order
  the guide's builders apply them), so those rows become full lower-triangular
  rows;
* the diagonal block is then forced on when asked (XAttention guide,
  "algorithm flow", phase 3: the causal diagonal block is always kept).  The
  guide's own test instead forces key-block column 0 through its scores and
  does not force the diagonal, which ``force_diagonal=False`` reproduces.

Compaction (the list form of the guide's §4.4 loop bound and block skip):
row (b, h, i) lists, ascending, every key block j with a nonzero mask byte and
j <= i when causal; ``cnt`` is the list length; the rest of the row is -1.
"""
from __future__ import annotations

import numpy as np


def _finish(mask: np.ndarray, dense_last_two_rows: bool, force_diagonal: bool) -> np.ndarray:
    nb = mask.shape[-1]
    if dense_last_two_rows:
        mask[..., max(0, nb - 2):, :] = 1
    mask = np.tril(mask)  # keep j <= i on the last two axes
    if force_diagonal:
        d = np.arange(nb)
        mask[..., d, d] = 1
    return mask.astype(np.uint8)


def build_mask_topk(scores: np.ndarray, topk: int, dense_last_two_rows: bool = False,
                    force_diagonal: bool = True) -> np.ndarray:
    """scores float [B, H, nb, nb] -> uint8 0/1 mask [B, H, nb, nb]."""
    scores = np.asarray(scores)
    nb = scores.shape[-1]
    assert scores.shape[-2] == nb and 0 <= topk <= nb
    # Descending score; a stable sort keeps equal scores in column order.
    order = np.argsort(-scores, axis=-1, kind="stable")
    mask = np.zeros(scores.shape, dtype=np.uint8)
    np.put_along_axis(mask, order[..., :topk], 1, axis=-1)
    return _finish(mask, dense_last_two_rows, force_diagonal)


def build_mask_threshold(scores: np.ndarray, threshold: float, dense_last_two_rows: bool = False,
                         force_diagonal: bool = True) -> np.ndarray:
    """scores float [B, H, nb, nb] -> uint8 0/1 mask, kept where score > threshold."""
    scores = np.asarray(scores)
    assert scores.shape[-1] == scores.shape[-2]
    mask = (scores > np.float32(threshold)).astype(np.uint8)
    return _finish(mask, dense_last_two_rows, force_diagonal)


def mask_to_indices(mask: np.ndarray, is_causal: bool):
    """mask [B, H, nb, nb] (nonzero = selected) -> (idx int32 [B,H,nb,nb], cnt int32 [B,H,nb])."""
    mask = np.asarray(mask)
    B, H, nb, nb2 = mask.shape
    assert nb == nb2
    idx = np.full((B, H, nb, nb), -1, dtype=np.int32)
    cnt = np.zeros((B, H, nb), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                cols = np.flatnonzero(mask[b, h, i] != 0)
                if is_causal:
                    cols = cols[cols <= i]
                idx[b, h, i, :cols.size] = cols
                cnt[b, h, i] = cols.size
    return idx, cnt
