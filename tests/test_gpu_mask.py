"""GPU parity: mask builders and compaction must equal the oracle byte for byte."""
import numpy as np
import pytest

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import mask as om
from tests.gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu


def _gpu_mask(scores, cfg_kind, val, dense, diag):
    s = to_gpu(scores.astype(np.float32))
    if cfg_kind == "topk":
        m = bsa.bsattn_build_mask_topk(s, int(val), dense, diag)
    else:
        m = bsa.bsattn_build_mask_threshold(s, float(val), dense, diag)
    return m.cpu().numpy()


@pytest.mark.parametrize("name", ["P0", "P1", "C1", "C2", "C3", "C4"])
def test_config_masks(name):
    cfg = gen.CONFIGS[name]
    nb = cfg.nb
    shp = (cfg.B, cfg.H, nb, nb)
    scores = gen.prefill_scores(cfg, 0)
    val = cfg.topk if cfg.mask_kind == "topk" else cfg.threshold
    say(f"[mask] {name} {cfg.mask_kind}={val} shape={shp}")
    got = _gpu_mask(scores, cfg.mask_kind, val, cfg.dense_last_two_rows, cfg.force_diagonal)
    if cfg.mask_kind == "topk":
        want = om.build_mask_topk(scores, cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    else:
        want = om.build_mask_threshold(scores, cfg.threshold, cfg.dense_last_two_rows, cfg.force_diagonal)
    np.testing.assert_array_equal(got, want)
    causal_blocks = cfg.B * cfg.H * nb * (nb + 1) // 2
    say(f"  density {want.sum() / causal_blocks:.4f}")


@pytest.mark.parametrize("nb", [1, 2, 3, 63, 64, 65, 257, 300])
def test_topk_ties_and_sizes(nb):
    rng = np.random.default_rng(nb)
    scores = rng.integers(-2, 3, size=(2, 3, nb, nb)).astype(np.float32)
    scores[0, 0, :, ::2] = -0.0
    scores[0, 1, :, 1::2] = 0.0
    for topk in sorted({0, 1, min(3, nb), nb // 2, nb}):
        for dense in (False, True):
            for diag in (False, True):
                say(f"[mask] topk ties nb={nb} topk={topk} dense={dense} diag={diag}")
                got = _gpu_mask(scores, "topk", topk, dense, diag)
                np.testing.assert_array_equal(got, om.build_mask_topk(scores, topk, dense, diag))


def test_topk_long_rows_chunked():
    # rows longer than one LDS chunk of the ranking loop
    nb = 2100
    rng = np.random.default_rng(1)
    scores = rng.integers(0, 50, size=(1, 1, nb, nb)).astype(np.float32)
    say(f"[mask] topk nb={nb}")
    got = _gpu_mask(scores, "topk", 37, False, True)
    np.testing.assert_array_equal(got, om.build_mask_topk(scores, 37, False, True))


@pytest.mark.parametrize("nb", [1, 2, 7, 64, 129])
def test_threshold_sizes(nb):
    rng = np.random.default_rng(100 + nb)
    scores = rng.random((2, 2, nb, nb), dtype=np.float32)
    scores[..., 0] = np.float32(0.5)          # exact equality with the threshold is not kept
    for thr in (0.5, 0.9, -np.inf, np.inf):
        for dense in (False, True):
            for diag in (False, True):
                say(f"[mask] threshold nb={nb} t={thr} dense={dense} diag={diag}")
                got = _gpu_mask(scores, "threshold", thr, dense, diag)
                np.testing.assert_array_equal(got, om.build_mask_threshold(scores, thr, dense, diag))


@pytest.mark.parametrize("nb", [1, 5, 64, 65, 130, 300])
@pytest.mark.parametrize("causal", [True, False])
def test_compaction(nb, causal):
    rng = np.random.default_rng(nb * 7 + causal)
    mask = (rng.random((2, 3, nb, nb)) < 0.35).astype(np.uint8)
    mask *= rng.integers(1, 256, size=mask.shape).astype(np.uint8)   # any nonzero byte selects
    mask[0, 0, -1, :] = 0
    say(f"[compact] nb={nb} causal={causal}")
    idx, cnt = bsa.bsattn_mask_to_indices(to_gpu(mask), causal)
    want_idx, want_cnt = om.mask_to_indices(mask, causal)
    np.testing.assert_array_equal(cnt.cpu().numpy(), want_cnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), want_idx)
