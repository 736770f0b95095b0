"""GPU parity: the fused mask-build + forward entry points.

bsattn_fwd_topk / bsattn_fwd_threshold must write the same mask bytes as the
stand-alone builders (and as the oracle), and produce outputs bit-identical
to bsattn_fwd on that mask: the same block lists in the same order, and the
same split of causal rows of more than 128 key blocks into two halves and a
merge.  The chunk entry with Sq = Sk, which runs every row whole, agrees with
both within the output tolerance (and bit for bit where no row splits)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _both(q, k, v, scores, cfg_kind, param, dense2, diag, causal):
    s = to_gpu(scores)
    if cfg_kind == "topk":
        m = bsa.bsattn_build_mask_topk(s, param, dense2, diag)
        fused, fm = bsa.bsattn_fwd_topk(q, k, v, s, param, dense2, diag, causal, write_mask=True)
    else:
        m = bsa.bsattn_build_mask_threshold(s, param, dense2, diag)
        fused, fm = bsa.bsattn_fwd_threshold(q, k, v, s, param, dense2, diag, causal, write_mask=True)
    ref = bsa.bsattn_fwd(q, k, v, m, causal)
    whole = bsa.bsattn_fwd_chunk(q, k, v, m, causal)
    check_close(gpu_bf16_to_f64(ref), gpu_bf16_to_f64(whole), "bsattn_fwd against whole rows")
    if q.shape[2] <= 128 * 64 or not causal:   # no row can split
        assert torch.equal(ref.view(torch.int16), whole.view(torch.int16))
    return m, ref, fm, fused


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "P0", "P1"])
def test_configs_match_the_two_launch_path(name):
    cfg = gen.CONFIGS[name]
    inp = gen.prefill_inputs(cfg, 0)
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    param = cfg.topk if cfg.mask_kind == "topk" else cfg.threshold
    say(f"[fused] {name} {cfg.mask_kind} {param}")
    m, ref, fm, fused = _both(q, k, v, inp["scores"], cfg.mask_kind, param,
                              cfg.dense_last_two_rows, cfg.force_diagonal, cfg.is_causal)
    assert torch.equal(fm, m)
    assert torch.equal(fused.view(torch.int16), ref.view(torch.int16))
    if cfg.nb <= 64:
        want = (om.build_mask_topk(inp["scores"], param, cfg.dense_last_two_rows, cfg.force_diagonal)
                if cfg.mask_kind == "topk" else
                om.build_mask_threshold(inp["scores"], param, cfg.dense_last_two_rows, cfg.force_diagonal))
        np.testing.assert_array_equal(fm.cpu().numpy(), want)


@pytest.mark.parametrize("S,D", [(40, 64), (64, 128), (200, 64), (1000, 128)])
@pytest.mark.parametrize("topk", [0, 1, 3, None])
def test_topk_edges_and_ties(S, D, topk):
    rng = np.random.default_rng(S + D)
    B, H = 2, 3
    nb = -(-S // 64)
    tk = nb if topk is None else min(topk, nb)
    # few distinct values: many ties, plus signed zeros
    scores = rng.integers(-2, 3, size=(B, H, nb, nb)).astype(np.float32) * 0.5
    scores[..., 0, 0] = -0.0
    q, k, v = (to_gpu_bf16(gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32)))
               for _ in range(3))
    for dense2 in (False, True):
        for diag in (True, False):
            for causal in (True, False):
                say(f"[fused] topk S={S} D={D} k={tk} dense2={dense2} diag={diag} causal={causal}")
                m, ref, fm, fused = _both(q, k, v, scores, "topk", tk, dense2, diag, causal)
                assert torch.equal(fm, m)
                assert torch.equal(fused.view(torch.int16), ref.view(torch.int16))
                np.testing.assert_array_equal(fm.cpu().numpy(), om.build_mask_topk(scores, tk, dense2, diag))


@pytest.mark.parametrize("thr", [-1e30, 0.3, 0.99, 1e30])
def test_threshold_edges(thr):
    rng = np.random.default_rng(5)
    B, H, S, D = 1, 4, 450, 64
    nb = -(-S // 64)
    scores = rng.random((B, H, nb, nb), dtype=np.float32)
    q, k, v = (to_gpu_bf16(gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32)))
               for _ in range(3))
    say(f"[fused] threshold {thr}")
    m, ref, fm, fused = _both(q, k, v, scores, "threshold", thr, True, True, True)
    assert torch.equal(fm, m)
    assert torch.equal(fused.view(torch.int16), ref.view(torch.int16))
    np.testing.assert_array_equal(fm.cpu().numpy(), om.build_mask_threshold(scores, thr, True, True))


def test_without_mask_output():
    cfg = gen.CONFIGS["C1"]
    inp = gen.prefill_inputs(cfg, 0)
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    s = to_gpu(inp["scores"])
    say("[fused] no mask output")
    a = bsa.bsattn_fwd_topk(q, k, v, s, cfg.topk)
    b, _ = bsa.bsattn_fwd_topk(q, k, v, s, cfg.topk, write_mask=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("kind", ["topk", "threshold"])
@pytest.mark.parametrize("S,H,D", [(8320, 8, 128), (8300, 4, 64)])
def test_long_rows_split_like_bsattn_fwd(kind, S, H, D):
    """Rows of more than 128 selected key blocks split in the fused forms too.
    Threshold: heavy rows 128 and 129 (129 and 130 blocks, and on odd heads a
    row 129 of exactly 128 that stays whole), light rows elsewhere, and a last
    head with no long row (its helpers have nothing to do).  Top-k with
    k = 129 keeps nearly every causal block, so rows 128 and 129 are long on
    every head.  The output matches bsattn_fwd bit for bit (one workspace
    serves both calls) and the oracle on the rows past block 127."""
    nb = -(-S // 64)
    rng = np.random.default_rng(S + H + D)
    scores = rng.random((1, H, nb, nb), dtype=np.float32) * 0.5    # all below 0.9: light rows
    for h in range(H - 1):
        scores[0, h, 128, :129] = 1.0
        scores[0, h, 129, :130] = 1.0
        if h % 2:
            scores[0, h, 129, [3, 77]] = 0.0
    scores[0, :, np.arange(nb), np.arange(nb)] = 1.0
    qkv = {n: gen.f32_to_bf16_bits(rng.standard_normal((1, H, S, D), dtype=np.float32))
           for n in ("q", "k", "v")}
    q, k, v = (to_gpu_bf16(qkv[n]) for n in ("q", "k", "v"))
    ws = torch.empty(bsa.bsattn_fwd_workspace_bytes(1, H, S, D), dtype=torch.uint8, device="cuda")
    s = to_gpu(scores)
    if kind == "topk":
        param, want_mask = 129, om.build_mask_topk(scores, 129, False, True)
        fused, fm = bsa.bsattn_fwd_topk(q, k, v, s, param, False, True, True, write_mask=True,
                                        workspace=ws)
    else:
        param, want_mask = 0.9, om.build_mask_threshold(scores, 0.9, False, True)
        fused, fm = bsa.bsattn_fwd_threshold(q, k, v, s, param, False, True, True, write_mask=True,
                                             workspace=ws)
    say(f"[fused] long rows {kind} S={S} H={H} D={D} blocks={int(want_mask.sum())}")
    np.testing.assert_array_equal(fm.cpu().numpy(), want_mask)
    assert int(want_mask[0, 0, 129].sum()) == 130
    ref = bsa.bsattn_fwd(q, k, v, fm, True, workspace=ws)
    assert torch.equal(fused.view(torch.int16), ref.view(torch.int16))
    rows = sorted(set(range(127 * 64, S)) | {0, S // 2})
    x = {n: gen.bf16_bits_to_f64(qkv[n]) for n in qkv}
    want = np.stack([oa.prefill_head_rows(x["q"][0, h], x["k"][0, h], x["v"][0, h], want_mask[0, h],
                                          True, rows) for h in range(H)])
    check_close(gpu_bf16_to_f64(fused)[0][:, rows], want, f"fused {kind} long rows S{S} H{H} D{D}")


@pytest.mark.parametrize("kind", ["topk", "threshold"])
@pytest.mark.parametrize("causal", [True, False])
def test_past_256_blocks_runs_as_two_launches(kind, causal):
    """Past 256 key blocks a row no longer fits the one-launch prologue: the
    call builds the mask into mask_out and runs the mask-row forward on it,
    with the builder's mask bytes and bsattn_fwd's output."""
    B, H, S, D = 1, 2, 64 * 260 - 20, 64
    nb = -(-S // 64)
    rng = np.random.default_rng(260 + causal)
    scores = rng.random((B, H, nb, nb), dtype=np.float32)
    qkv = {n: gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
           for n in ("q", "k", "v")}
    q, k, v = (to_gpu_bf16(qkv[n]) for n in ("q", "k", "v"))
    s = to_gpu(scores)
    say(f"[fused] {kind} past 256 blocks: nb={nb} causal={causal}")
    if kind == "topk":
        fused, fm = bsa.bsattn_fwd_topk(q, k, v, s, 12, True, True, causal, write_mask=True)
        bare = bsa.bsattn_fwd_topk(q, k, v, s, 12, True, True, causal)
        want_mask = om.build_mask_topk(scores, 12, True, True)
    else:
        fused, fm = bsa.bsattn_fwd_threshold(q, k, v, s, 0.95, True, True, causal, write_mask=True)
        bare = bsa.bsattn_fwd_threshold(q, k, v, s, 0.95, True, True, causal)
        want_mask = om.build_mask_threshold(scores, 0.95, True, True)
    np.testing.assert_array_equal(fm.cpu().numpy(), want_mask)
    ref = bsa.bsattn_fwd(q, k, v, fm, causal)
    assert torch.equal(fused.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(bare.view(torch.int16), ref.view(torch.int16))
    rows = [0, 63, 64 * 128 + 5, 64 * 200, S - 65, S - 1]
    x = {n: gen.bf16_bits_to_f64(qkv[n]) for n in qkv}
    want = np.stack([oa.prefill_head_rows(x["q"][0, h], x["k"][0, h], x["v"][0, h], want_mask[0, h],
                                          causal, rows) for h in range(H)])
    check_close(gpu_bf16_to_f64(fused)[0][:, rows], want, f"fused {kind} nb={nb} causal={causal}")
