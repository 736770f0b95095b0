"""GPU parity: the fused mask-build + forward entry points.

bsattn_fwd_topk / bsattn_fwd_threshold must write the same mask bytes as the
stand-alone builders (and as the oracle), and produce outputs bit-identical
to the mask-driven forward pass on that mask when it runs every row whole
(the chunk entry with Sq = Sk: the same block lists in the same order).
bsattn_fwd, which splits causal rows of more than 128 key blocks in two,
agrees with them within the output tolerance."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
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
    ref = bsa.bsattn_fwd_chunk(q, k, v, m, causal)
    split = bsa.bsattn_fwd(q, k, v, m, causal)
    check_close(gpu_bf16_to_f64(split), gpu_bf16_to_f64(ref), "bsattn_fwd against whole rows")
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
