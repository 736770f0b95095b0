"""XAttention block-importance estimator oracle — test infrastructure only.

Plain numpy float64 statement of the estimator that produces block scores
upstream of the block mask (XAttention guide: "algorithm flow" phases 1-3).
Only ``tests/``, the smoke check and the bench's CPU-baseline leg may use it.

1. Stride reshape, inverse mode (XAttention guide, stride-reshape section):
   with stride s, reshaped key row t' is the concatenation of key rows
   t's, t's+1, ..., t's+s-1 (forward interleave); reshaped query row r' is
   the concatenation of query rows r's+s-1, r's+s-2, ..., r's (reverse
   interleave).  Lengths shrink by s, the feature dimension grows to s*D.
2. Block estimate (same guide, the fused reshape-GEMM and the softmax +
   block-sum kernel descriptions): logits Q'K'^T, a row softmax over the
   reshaped keys, then for every (query block, key block) the sum of the
   softmax weights over the block's reshaped rows and columns.
3. Block selection (same guide, block-selection section): per query-block
   row, the row total, the required mass threshold * total, the sink column
   and the diagonal column kept, the other columns ranked by weight and kept
   by cumulative weight.

Readings (the page leaves these open or states them inconsistently):

* logit scale: the reshaped dot product sums s token-pair products, so it is
  divided by s as well as sqrt(D), and by the ``norm`` parameter of the key
  parameter table: logit = (q'.k') / (sqrt(D) * s * norm).
* causal: on the reshaped grid, key t' is visible to query r' when
  t' <= r' + (Sk - Sq) / s (queries are the last Sq of Sk positions); the
  diagonal reshaped pair is kept whole, which is the approximation of the
  causal diagonal the inverse interleave is for.
* the block is the forward kernel's block, 64 tokens, i.e. 64 / s reshaped
  rows and columns (the page's sparse kernel fixes 128 for its own library).
* selection keeps a column while the weight ranked above it (the exclusive
  cumulative sum) is still below the required mass, i.e. the smallest ranked
  prefix that reaches it.  This is what the flow chart (weights added until
  they reach the threshold's share of the total) and the worked example (row
  0.05 0.30 0.40 0.15 0.10 at 0.9 keeps four blocks) say; testing the
  inclusive cumulative sum against the required mass, as the listing does,
  would keep three there.
* the total includes the kept sink and diagonal weights; their weights are
  zeroed before ranking, as the listing does.  Ties rank the lower column
  first.  Sums and the comparison are float64: the total accumulates in
  ascending column order and the ranked sum in rank order, one term at a time.
* sink and diagonal are flags (the listing always keeps both; the parameter
  table lists them as options); columns after the diagonal are then dropped
  on the causal path (they carry no weight and the causal forward never
  visits them).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


def stride_reshape(q: np.ndarray, k: np.ndarray, stride: int):
    """q [..., Sq, D], k [..., Sk, D] -> (Q' [..., Sq/s, s*D], K' [..., Sk/s, s*D])."""
    s = stride
    assert q.shape[-2] % s == 0 and k.shape[-2] % s == 0
    kr = np.concatenate([k[..., j::s, :] for j in range(s)], axis=-1)
    qr = np.concatenate([q[..., (s - 1 - j)::s, :] for j in range(s)], axis=-1)
    return qr, kr


def block_sums(q: np.ndarray, k: np.ndarray, stride: int, norm: float = 1.0,
               causal: bool = True) -> np.ndarray:
    """q [B, H, Sq, D], k [B, H, Sk, D] -> float64 [B, H, ceil(Sq/64), ceil(Sk/64)]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    Sq, D = q.shape[-2], q.shape[-1]
    Sk = k.shape[-2]
    s = stride
    assert Sq <= Sk and BLOCK % s == 0
    qr, kr = stride_reshape(q, k, s)
    logits = (qr @ np.swapaxes(kr, -1, -2)) / (np.sqrt(D) * s * norm)
    rq, rk = Sq // s, Sk // s
    if causal:
        past = (Sk - Sq) // s
        visible = np.arange(rk)[None, :] <= np.arange(rq)[:, None] + past
        logits = np.where(visible, logits, -np.inf)
    mx = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - mx)
    p /= p.sum(axis=-1, keepdims=True)
    b = BLOCK // s
    nbq, nbk = -(-Sq // BLOCK), -(-Sk // BLOCK)
    out = np.zeros(q.shape[:-2] + (nbq, nbk))
    for qi in range(nbq):
        for ki in range(nbk):
            out[..., qi, ki] = p[..., qi * b:(qi + 1) * b, ki * b:(ki + 1) * b].sum(axis=(-1, -2))
    return out


def _sequential_sum(x: np.ndarray) -> float:
    acc = 0.0
    for v in x:
        acc += float(v)
    return acc


def find_blocks_row(x: np.ndarray, threshold: float, sink: int | None, diag: int | None,
                    causal_last: int | None) -> np.ndarray:
    """One row of block weights (float32 values) -> uint8 0/1 selection.

    sink / diag: the kept columns (None: not kept); causal_last: the last
    column a causal row may keep (None: all)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    n = x.shape[0]
    total = _sequential_sum(x)                      # ascending column order
    required = float(np.float32(threshold)) * total
    keep = np.zeros(n, bool)
    for c in (sink, diag):
        if c is not None and 0 <= c < n:
            keep[c] = True
    other = np.where(keep, 0.0, x)
    order = np.argsort(-other, kind="stable")      # weight descending, lower column first
    ranked_before = 0.0
    for c in order:                                 # rank order, one term at a time
        if ranked_before < required:
            keep[c] = True
        ranked_before += other[c]
    if causal_last is not None:
        keep[causal_last + 1:] = False
    return keep.astype(np.uint8)


def find_blocks(sums: np.ndarray, threshold: float, keep_sink: bool = True,
                keep_diagonal: bool = True, causal: bool = True) -> np.ndarray:
    """sums float32 [B, H, nbq, nbk] -> uint8 0/1 mask; query blocks are the last nbq of nbk."""
    sums = np.asarray(sums, np.float32)
    nbq, nbk = sums.shape[-2], sums.shape[-1]
    assert nbq <= nbk
    past = nbk - nbq
    out = np.zeros(sums.shape, np.uint8)
    for idx in np.ndindex(*sums.shape[:-2]):
        for i in range(nbq):
            d = i + past
            out[idx + (i,)] = find_blocks_row(sums[idx + (i,)], threshold,
                                              0 if keep_sink else None,
                                              d if keep_diagonal else None,
                                              d if causal else None)
    return out


def estimate_mask(q, k, stride: int = 8, norm: float = 1.0, threshold: float = 0.9,
                  keep_sink: bool = True, keep_diagonal: bool = True, causal: bool = True):
    """The whole estimator: (block sums float64, mask uint8).  The selection
    runs on the float32 rounding of the block sums, the precision the block
    sums are handed over in."""
    bs = block_sums(q, k, stride, norm, causal)
    return bs, find_blocks(bs.astype(np.float32), threshold, keep_sink, keep_diagonal, causal)
