"""GPU: the kernels read only what the selection names.

Every key/value row that no selected block of its (batch, head) holds is set
to NaN on the device, so any use of such a row -- even with a zero weight,
since 0 * NaN is NaN -- makes an output non-finite.  The outputs are then
compared with the oracle on the same inputs without the NaNs (the oracle
reads only selected blocks' rows, TileLang block-sparse Flash-Attention
guide §4.4 for the forward's block skip, §6 for the decode's block indices).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

NAN_BITS = np.uint16(0x7FC0)   # bfloat16 quiet NaN


@pytest.mark.parametrize("S,D,causal,density", [
    (4096 + 37, 64, True, 0.3), (4096 + 37, 128, False, 0.3), (2048, 128, True, 0.6),
    (9000, 128, True, 0.97),   # rows past 128 blocks: the long-row split and its merge
    (9000, 64, True, 0.97),
])
def test_prefill_reads_only_selected_blocks(S, D, causal, density):
    B, H = 1, 2
    rng = np.random.default_rng(S + D + int(causal) + int(100 * density))
    nb = -(-S // 64)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
    m = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    kp, vp = k.copy(), v.copy()
    for h in range(H):
        # key blocks no row of this head selects (never block 0, so most rows see a key)
        cut = rng.choice(np.arange(1, nb), size=max(1, nb // 10), replace=False)
        m[0, h, :, cut] = 0
        for j in cut:
            kp[0, h, 64 * j:64 * j + 64] = NAN_BITS
            vp[0, h, 64 * j:64 * j + 64] = NAN_BITS
    say(f"[poison-prefill] S={S} D={D} causal={causal} density={density} blocks={int(m.sum())}")
    got = gpu_bf16_to_f64(bsa.bsattn_fwd(to_gpu_bf16(q), to_gpu_bf16(kp), to_gpu_bf16(vp),
                                         to_gpu(m), causal))
    f = gen.bf16_bits_to_f64
    want = oa.prefill(f(q), f(k), f(v), m, causal)
    check_close(got, want, f"poisoned prefill S{S} D{D} c{causal}")


def _poison_packed(inp, Hkv):
    """k, v [T, Hkv, D] with every (token, KV head) row outside its
    sequence's selected blocks set to NaN."""
    cu, idx = inp["cu_seqlens_k"], inp["block_indices"]
    kp, vp = inp["k"].copy(), inp["v"].copy()
    for b in range(len(cu) - 1):
        L = int(cu[b + 1] - cu[b])
        blk = np.arange(L) // 64
        for h in range(Hkv):
            keep = np.isin(blk, idx[b, h][idx[b, h] >= 0])
            rows = cu[b] + np.nonzero(~keep)[0]
            kp[rows, h] = NAN_BITS
            vp[rows, h] = NAN_BITS
    return kp, vp


def _poison_paged(inp, Hkv):
    """The paged cache with every row that no selected block of its (batch,
    KV head) holds set to NaN: unused pages, rows past a sequence's end, and
    unselected blocks."""
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    ps, table, idx = int(inp["page_size"]), inp["block_table"], inp["block_indices"]
    used = np.zeros(kc.shape[0], bool)
    for b in range(table.shape[0]):
        L = int(inp["cache_seqlens"][b])
        for lp, page in enumerate(table[b]):
            if page < 0:
                continue
            used[page] = True
            t = lp * ps + np.arange(ps)
            past = t >= L
            kc[page, past] = NAN_BITS
            vc[page, past] = NAN_BITS
            for h in range(Hkv):
                off = ~np.isin(t // 64, idx[b, h][idx[b, h] >= 0]) & ~past
                kc[page, off, h] = NAN_BITS
                vc[page, off, h] = NAN_BITS
    kc[~used] = NAN_BITS
    vc[~used] = NAN_BITS
    return kc, vc


@pytest.mark.parametrize("cfg", [
    gen.CONFIGS["P2"],
    gen.custom_decode(5, 16, 2, 64, 100, 3000, max_selected_blocks=16, sparse_ratio=0.7),
    gen.custom_decode(3, 64, 1, 128, 700, 5000, max_selected_blocks=24, sparse_ratio=0.6),
], ids=["P2", "ragged-D64", "G64"])
@pytest.mark.parametrize("form", ["index", "mask", "paged"])
def test_decode_reads_only_selected_blocks(cfg, form):
    inp = gen.decode_inputs(cfg, 5)
    x = {n: gen.bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v")}
    want = oa.decode_gqa(x["q"], x["k"], x["v"], inp["cu_seqlens_k"], inp["block_indices"])
    q = to_gpu_bf16(inp["q"])
    say(f"[poison-decode] {cfg.name} form={form} total_k={int(inp['cu_seqlens_k'][-1])}")
    for ns in (1, 3):
        if form == "paged":
            pin = gen.decode_paged_inputs(cfg, 5, base=inp)
            kc, vc = _poison_paged(pin, cfg.Hkv)
            out = bsa.bsattn_decode_gqa_paged(q, to_gpu_bf16(kc), to_gpu_bf16(vc),
                                              to_gpu(pin["cache_seqlens"]), to_gpu(pin["block_table"]),
                                              to_gpu(pin["block_indices"]), num_splits=ns)
        else:
            kp, vp = _poison_packed(inp, cfg.Hkv)
            k, v, cu = to_gpu_bf16(kp), to_gpu_bf16(vp), to_gpu(inp["cu_seqlens_k"])
            if form == "index":
                out = bsa.bsattn_decode_gqa(q, k, v, cu, to_gpu(inp["block_indices"]), num_splits=ns)
            else:
                mi = gen.decode_mask_inputs(cfg, 5, base=inp)
                out = bsa.bsattn_decode_gqa_mask(q, k, v, cu, to_gpu(mi["block_mask"]), num_splits=ns)
        check_close(gpu_bf16_to_f64(out), want, f"poisoned decode {cfg.name} {form} ns{ns}")


@pytest.mark.parametrize("kind", ["topk", "threshold"])
@pytest.mark.parametrize("S,D,causal,dense", [(4096 + 37, 64, True, False), (2048, 128, False, False),
                                               (9000, 128, True, True)])
def test_fused_reads_only_selected_blocks(kind, S, D, causal, dense):
    """The one-launch forms select each row from the block scores in the
    kernel.  Without the forced diagonal, key blocks whose scores are far
    below every other score (and below the threshold) are never selected, so
    their K/V rows can hold NaN; S = 9000 also takes the long-row split."""
    B, H = 1, 2
    rng = np.random.default_rng(S + D + int(causal) + (kind == "topk"))
    nb = -(-S // 64)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
    scores = rng.standard_normal((B, H, nb, nb), dtype=np.float32)
    kp, vp = k.copy(), v.copy()
    for h in range(H):
        cut = rng.choice(np.arange(1, nb), size=3 if dense else max(1, nb // 10), replace=False)
        scores[0, h, :, cut] = -1e30
        for j in cut:
            kp[0, h, 64 * j:64 * j + 64] = NAN_BITS
            vp[0, h, 64 * j:64 * j + 64] = NAN_BITS
    # fewer than the uncut columns; N(0, 1) scores above the threshold.  Dense:
    # rows past 128 blocks, which split
    topk, thr = (nb - 3, -4.0) if dense else (nb // 2, 0.0)
    if kind == "topk":
        m = om.build_mask_topk(scores, topk, False, False)
    else:
        m = om.build_mask_threshold(scores, thr, False, False)
    say(f"[poison-fused] {kind} S={S} D={D} causal={causal} blocks={int(m.sum())}")
    args = (to_gpu_bf16(q), to_gpu_bf16(kp), to_gpu_bf16(vp), to_gpu(scores))
    if kind == "topk":
        got, gm = bsa.bsattn_fwd_topk(*args, topk, False, False, causal, write_mask=True)
    else:
        got, gm = bsa.bsattn_fwd_threshold(*args, thr, False, False, causal, write_mask=True)
    assert np.array_equal(gm.cpu().numpy(), m)
    f = gen.bf16_bits_to_f64
    want = oa.prefill(f(q), f(k), f(v), m, causal)
    check_close(gpu_bf16_to_f64(got), want, f"poisoned fused {kind} S{S} D{D} c{causal}")
