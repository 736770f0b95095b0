"""Seeded synthetic workloads for block-sparse attention (host side, numpy only).

This module draws random inputs and nothing else: it holds none of the
attention, mask or split arithmetic.  The same arrays feed the CPU oracle
(``oracle/``) and the HIP library, so both sides see identical data.

Each tensor gets its own child stream ``np.random.default_rng([seed, tag])``
with the tags below; draws are float32 and, where the workload says so,
rounded to bfloat16 (round to nearest even) on the host.  bfloat16 tensors
travel as their uint16 bit patterns; ``bf16_bits_to_f64`` widens them exactly.

Workload shapes follow the pages on block-sparse attention:

* TileLang block-sparse Flash-Attention guide, §5 (test: B1 H1 S256 D64,
  top-2 with the first key-block column forced by a score of 100) and §9.3
  (benchmark default [4, 2, 256, 64, 2, 64]);
* the same guide, §9.2 and §9.4 (decode: 32 query heads over 8 KV heads,
  D 128, sparse ratio 0.8, regression run at batch 1 and KV length 2048);
* the prefill and decode configurations this library is measured on (see
  ``CONFIGS``), whose value distributions are stated there.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

BLOCK = 64

TAG_SCORES, TAG_Q, TAG_K, TAG_V, TAG_LENS, TAG_INDICES, TAG_PAGES = 0, 1, 2, 3, 4, 5, 6


def child_rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction (normal / uniform draws)."""
    # In uint32: for finite inputs (bits <= 0xFF7FFFFF) adding at most 0x8000
    # cannot wrap.
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def nblocks(n: int, block: int = BLOCK) -> int:
    return -(-int(n) // block)


# --------------------------------------------------------------------------
# prefill workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    S: int
    D: int
    mask_kind: str            # "topk" or "threshold"
    topk: int = 0
    threshold: float = 0.0
    scores_dist: str = "normal"   # "normal" N(0,1) or "uniform" U(0,1)
    qkv_scale: float = 1.0
    dense_last_two_rows: bool = False
    force_diagonal: bool = True
    force_first_column: bool = False   # score 100 in key-block column 0
    is_causal: bool = True

    @property
    def nb(self) -> int:
        return nblocks(self.S)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    len_lo: int
    len_hi: int               # inclusive
    max_selected_blocks: int = 64
    sparse_ratio: float = 0.8


CONFIGS: Dict[str, object] = {
    # C1: B1 H2 S512 D64, scores N(0,1), top-3 then tril, diagonal forced; seed 0.
    "C1": PrefillConfig("C1", 1, 2, 512, 64, "topk", topk=3),
    # C2: B2 H16 S4096 D64, top-16 of N(0,1) block scores, tril, diagonal forced.
    "C2": PrefillConfig("C2", 2, 16, 4096, 64, "topk", topk=16),
    # C3: B1 H32 S16384 D128, U(0,1) scores > 0.92 (about 10% of causal blocks),
    # last two block rows dense, tril, diagonal forced.
    "C3": PrefillConfig("C3", 1, 32, 16384, 128, "threshold", threshold=0.92,
                        scores_dist="uniform", dense_last_two_rows=True),
    # C4: B4 H32 S8192 D128, Q/K/V N(0,1)*0.5, top-32, last two rows dense.
    "C4": PrefillConfig("C4", 4, 32, 8192, 128, "topk", topk=32, qkv_scale=0.5,
                        dense_last_two_rows=True),
    # C5: decode, batch 8, 32 query heads over 8 KV heads, D 128, KV lengths
    # U[4096, 32768], up to 64 selected 64-token blocks per (batch, kv head).
    "C5": DecodeConfig("C5", 8, 32, 8, 128, 4096, 32768),
    # P0: the guide's own prefill test (section 5): top-2, column 0 forced by a
    # score of 100, no diagonal forcing.
    "P0": PrefillConfig("P0", 1, 1, 256, 64, "topk", topk=2, force_diagonal=False,
                        force_first_column=True),
    # P1: the guide's benchmark default (section 9.3).
    "P1": PrefillConfig("P1", 4, 2, 256, 64, "topk", topk=2),
    # P2: the guide's decode regression size (section 9.4), block 64 here.
    "P2": DecodeConfig("P2", 1, 32, 8, 128, 2048, 2048),
}


def prefill_scores(cfg: PrefillConfig, seed: int = 0) -> np.ndarray:
    """Block importance scores, float32 [B, H, nb, nb]."""
    nb = cfg.nb
    shp = (cfg.B, cfg.H, nb, nb)
    g = child_rng(seed, TAG_SCORES)
    if cfg.scores_dist == "normal":
        scores = g.standard_normal(shp, dtype=np.float32)
    elif cfg.scores_dist == "uniform":
        scores = g.random(shp, dtype=np.float32)
    else:
        raise ValueError(cfg.scores_dist)
    if cfg.force_first_column:
        scores[..., 0] = np.float32(100.0)
    return scores


def prefill_qkv(cfg: PrefillConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """q, k, v as bfloat16 bits [B, H, S, D]."""
    out = {}
    qkv_shape = (cfg.B, cfg.H, cfg.S, cfg.D)
    for name, tag in (("q", TAG_Q), ("k", TAG_K), ("v", TAG_V)):
        x = child_rng(seed, tag).standard_normal(qkv_shape, dtype=np.float32)
        if cfg.qkv_scale != 1.0:
            x *= np.float32(cfg.qkv_scale)
        out[name] = f32_to_bf16_bits(x)
    return out


def prefill_inputs(cfg: PrefillConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """Scores (float32 [B,H,nb,nb]) and q/k/v (bf16 bits [B,H,S,D])."""
    out = {"scores": prefill_scores(cfg, seed)}
    out.update(prefill_qkv(cfg, seed))
    return out


def decode_inputs(cfg: DecodeConfig, seed: int = 0) -> Dict[str, np.ndarray]:
    """Packed-KV decode inputs.

    q bf16 [B,Hq,D]; k, v bf16 [total_k, Hkv, D] packed by ``cu_seqlens_k``
    (int32 [B+1]); ``block_indices`` int32 [B, Hkv, max_selected_blocks].

    Per sequence the number of selected blocks is
    ``min(max_selected_blocks, max(1, ceil((1 - sparse_ratio) * nb_b)))``.
    The last block ``nb_b - 1`` is always selected; the others are drawn
    uniformly without replacement from ``[0, nb_b - 1)``; each list is sorted
    descending (most recent first) and padded with -1.
    """
    lens = child_rng(seed, TAG_LENS).integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.B)
    lens = lens.astype(np.int64)
    cu = np.zeros(cfg.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    g_idx = child_rng(seed, TAG_INDICES)
    ms = cfg.max_selected_blocks
    idx = np.full((cfg.B, cfg.Hkv, ms), -1, dtype=np.int32)
    for b in range(cfg.B):
        nbb = nblocks(int(lens[b]))
        nsel = min(ms, max(1, math.ceil((1.0 - cfg.sparse_ratio) * nbb - 1e-9)))
        for h in range(cfg.Hkv):
            rest = g_idx.choice(nbb - 1, size=nsel - 1, replace=False) if nsel > 1 else np.zeros(0, np.int64)
            sel = np.concatenate([[nbb - 1], rest]).astype(np.int32)
            sel = np.sort(sel)[::-1]
            idx[b, h, :nsel] = sel
    out = {"lens": lens, "cu_seqlens_k": cu, "block_indices": idx}
    for name, tag, shape in (("q", TAG_Q, (cfg.B, cfg.Hq, cfg.D)),
                             ("k", TAG_K, (total, cfg.Hkv, cfg.D)),
                             ("v", TAG_V, (total, cfg.Hkv, cfg.D))):
        out[name] = f32_to_bf16_bits(child_rng(seed, tag).standard_normal(shape, dtype=np.float32))
    return out


def decode_mask_inputs(cfg: DecodeConfig, seed: int = 0,
                       base: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """The same workload in mask form: ``block_mask`` uint8 [B, Hkv, num_blocks]
    with num_blocks = the longest sequence's block count; column j is 1 when
    the index form selects block j (same draws as ``decode_inputs``, or the
    already generated ``base``)."""
    out = dict(base) if base is not None else decode_inputs(cfg, seed)
    nbk = max(nblocks(int(x)) for x in out["lens"])
    bm = np.zeros((cfg.B, cfg.Hkv, nbk), dtype=np.uint8)
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            sel = out["block_indices"][b, h]
            bm[b, h, sel[sel >= 0]] = 1
    out["block_mask"] = bm
    return out


def decode_paged_inputs(cfg: DecodeConfig, seed: int = 0, page_size: int = 256,
                        spare_pages: int = 16,
                        base: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """The same workload with K/V scattered into a paged cache.

    Sequence b's tokens fill ceil(len_b / page_size) pages taken from a seeded
    permutation of ``num_pages`` physical pages (``spare_pages`` of them stay
    unused and hold other draws): ``k_cache``/``v_cache`` bf16
    [num_pages, page_size, Hkv, D], ``block_table`` int32
    [B, max_blocks_per_seq] (-1 past a sequence's pages), ``cache_seqlens``
    int32 [B].  Token t of sequence b is row t % page_size of page
    block_table[b, t // page_size]; q and block_indices are those of
    ``decode_inputs`` (or of the already generated ``base``)."""
    out = dict(base) if base is not None else decode_inputs(cfg, seed)
    lens = out["lens"]
    per_seq = [-(-int(x) // page_size) for x in lens]
    mbps = max(per_seq)
    num_pages = sum(per_seq) + spare_pages
    g = child_rng(seed, TAG_PAGES)
    perm = g.permutation(num_pages)
    kc = np.empty((num_pages, page_size, cfg.Hkv, cfg.D), dtype=np.uint16)
    vc = np.empty_like(kc)
    fill = f32_to_bf16_bits(g.standard_normal((2, page_size, cfg.Hkv, cfg.D), dtype=np.float32))
    kc[:] = fill[0]
    vc[:] = fill[1]
    table = np.full((cfg.B, mbps), -1, dtype=np.int32)
    cu = out["cu_seqlens_k"]
    p = 0
    for b in range(cfg.B):
        for lp in range(per_seq[b]):
            page = int(perm[p])
            p += 1
            table[b, lp] = page
            t0, t1 = lp * page_size, min((lp + 1) * page_size, int(lens[b]))
            kc[page, :t1 - t0] = out["k"][cu[b] + t0:cu[b] + t1]
            vc[page, :t1 - t0] = out["v"][cu[b] + t0:cu[b] + t1]
    out.update({"k_cache": kc, "v_cache": vc, "block_table": table,
                "cache_seqlens": lens.astype(np.int32), "page_size": page_size})
    return out


def custom_prefill(B, H, S, D, mask_kind="topk", topk=2, threshold=0.5, **kw) -> PrefillConfig:
    return PrefillConfig(f"custom_B{B}H{H}S{S}D{D}", B, H, S, D, mask_kind, topk=topk,
                         threshold=threshold, **kw)


def custom_decode(B, Hq, Hkv, D, len_lo, len_hi, max_selected_blocks=64, sparse_ratio=0.8) -> DecodeConfig:
    return DecodeConfig(f"custom_dec_B{B}Hq{Hq}Hkv{Hkv}D{D}", B, Hq, Hkv, D, len_lo, len_hi,
                        max_selected_blocks, sparse_ratio)
