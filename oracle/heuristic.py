"""Split-count heuristic oracle (TileLang block-sparse Flash-Attention guide, §6.3).

Test infrastructure only (see ``oracle/__init__``).

Restated from the guide's description:

1. If the m-blocks alone nearly fill the machine (total_mblocks >= 0.8 x
   num_SMs), use one split — unless one KV head is larger than the assumed
   L2 (50 MiB), there are at least 2 x num_SMs m-blocks and the attention is
   neither causal nor local; then use ceil(size / L2) splits, capped at
   max_splits.
2. Else, with at most 4 KV blocks, use one split.
3. Else, for s in 1 .. min(max_splits, num_SMs, num_n_blocks), the wave
   efficiency is n_waves / ceil(n_waves) with n_waves = total_mblocks * s /
   num_SMs; return the smallest s whose efficiency reaches 85% of the best.

Readings: the garbled comparisons are >=, <= and >= respectively; "50 MB"
is taken as 50 * 2^20 bytes (it only matters in the non-causal branch,
which decode never takes).

For decode the guide calls it with is_causal_or_local = True, max_splits =
128 and size_one_kv_head = max_selected_blocks * block * (dim + dim_v) * 2.
With query heads grouped up to 64 per KV head, one (batch, KV head) pair is
one m-block: total_mblocks = B * Hq / min(64, Hq / Hkv), num_m_blocks = 1 and
num_n_blocks = max_selected_blocks.
"""
from __future__ import annotations

import math

L2_BYTES = 50 * 1024 * 1024


def num_splits_heuristic(total_mblocks: int, num_sms: int, num_n_blocks: int, num_m_blocks: int,
                         size_one_kv_head: int, is_causal_or_local: bool, max_splits: int) -> int:
    if total_mblocks >= 0.8 * num_sms:
        if (size_one_kv_head > L2_BYTES and num_m_blocks >= 2 * num_sms
                and not is_causal_or_local):
            return min(math.ceil(size_one_kv_head / L2_BYTES), max_splits)
        return 1
    if num_n_blocks <= 4:
        return 1
    cap = min(max_splits, num_sms, num_n_blocks)
    eff = []
    for s in range(1, cap + 1):
        n_waves = total_mblocks * s / num_sms
        eff.append(n_waves / math.ceil(n_waves))
    best = max(eff)
    for s, e in enumerate(eff, start=1):
        if e >= 0.85 * best:
            return s
    return 1


def decode_num_splits(B: int, Hq: int, Hkv: int, max_selected_blocks: int, D: int, num_cus: int,
                      block: int = 64) -> int:
    group = Hq // Hkv
    valid_block_h = min(64, group)
    total_mblocks = B * (Hq // valid_block_h)
    size_one_kv_head = max_selected_blocks * block * (D + D) * 2
    return num_splits_heuristic(total_mblocks, num_cus, max_selected_blocks, 1, size_one_kv_head,
                                True, 128)
