"""GPU parity at the two largest prefill workloads, every work item checked.

B1 H32 S16384 D128 (threshold mask, dense last two block rows: rows of more
than 128 key blocks split in two) and B4 H32 S8192 D128 (top-32, dense last
two rows) run at full size in the launch configuration the benchmark times.
Every (batch, head, query block) work item is compared with the oracle on
four of its rows — the first and last row of each 32-row wave group — so
every work-group, split halves included, meets the oracle (the block-sparse
guide's §5 reference check, restricted to rows the oracle computes one by
one).  The fused one-launch forms run on the same workloads and meet the
oracle on the same rows; their mask output is byte-exact.  A third workload,
B1 H32 S8192 D64 (top-32, dense last two rows), runs the D = 64 issue order
in which every head group's two heaviest rows go out two groups early."""
import functools

import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from tests.gpu_util import check_close, gpu_bf16_to_f64, parallel_map, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

ROWS_IN_BLOCK = (0, 31, 32, 63)


def _rows(S):
    nb = -(-S // 64)
    return np.array([64 * i + r for i in range(nb) for r in ROWS_IN_BLOCK if 64 * i + r < S], np.int64)


# four heads per XCD, two per group (2 MiB of K/V each at S8192 D64): two
# groups, so the look-ahead order is the one that runs
D64 = gen.custom_prefill(1, 32, 8192, 64, "topk", topk=32, dense_last_two_rows=True, qkv_scale=0.5)


@functools.lru_cache(maxsize=2)
def _case(name):
    """Inputs, the oracle's mask and the oracle's rows for every (b, h)."""
    cfg = D64 if name == "D64" else gen.CONFIGS[name]
    inp = gen.prefill_inputs(cfg, 0)
    if cfg.mask_kind == "topk":
        mask = om.build_mask_topk(inp["scores"], cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    else:
        mask = om.build_mask_threshold(inp["scores"], cfg.threshold, cfg.dense_last_two_rows,
                                       cfg.force_diagonal)
    rows = _rows(cfg.S)

    def one(bh):
        b, h = bh
        q, k, v = (gen.bf16_bits_to_f64(inp[n][b, h]) for n in ("q", "k", "v"))
        return oa.prefill_head_rows(q, k, v, mask[b, h], cfg.is_causal, rows)

    say(f"[prefill-full] {name}: oracle on {len(rows)} rows x {cfg.B * cfg.H} heads")
    want = parallel_map(one, [(b, h) for b in range(cfg.B) for h in range(cfg.H)])
    want = np.stack(want).reshape(cfg.B, cfg.H, len(rows), cfg.D)
    return cfg, inp, mask, rows, want


def _gather(out, rows):
    idx = torch.from_numpy(rows).to(out.device)
    return gpu_bf16_to_f64(out.index_select(2, idx))


@pytest.mark.parametrize("name", ["C3", "C4", "D64"])
def test_every_work_item_two_launch_path(name):
    cfg, inp, mask, rows, want = _case(name)
    say(f"[prefill-full] {name} builder + bsattn_fwd, B{cfg.B} H{cfg.H} S{cfg.S} D{cfg.D}")
    scores = to_gpu(inp["scores"])
    if cfg.mask_kind == "topk":
        m = bsa.bsattn_build_mask_topk(scores, cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    else:
        m = bsa.bsattn_build_mask_threshold(scores, cfg.threshold, cfg.dense_last_two_rows,
                                            cfg.force_diagonal)
    np.testing.assert_array_equal(m.cpu().numpy(), mask)
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    out = bsa.bsattn_fwd(q, k, v, m, cfg.is_causal)
    got = _gather(out, rows)
    check_close(got, want, f"{name} every item, rows {ROWS_IN_BLOCK} of each block")
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("name", ["C3", "C4"])
def test_every_work_item_fused_path(name):
    cfg, inp, mask, rows, want = _case(name)
    say(f"[prefill-full] {name} fused {cfg.mask_kind}, B{cfg.B} H{cfg.H} S{cfg.S} D{cfg.D}")
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    scores = to_gpu(inp["scores"])
    if cfg.mask_kind == "topk":
        out, m = bsa.bsattn_fwd_topk(q, k, v, scores, cfg.topk, cfg.dense_last_two_rows,
                                     cfg.force_diagonal, cfg.is_causal, write_mask=True)
    else:
        out, m = bsa.bsattn_fwd_threshold(q, k, v, scores, cfg.threshold, cfg.dense_last_two_rows,
                                          cfg.force_diagonal, cfg.is_causal, write_mask=True)
    np.testing.assert_array_equal(m.cpu().numpy(), mask)
    got = _gather(out, rows)
    check_close(got, want, f"{name} fused, every item, rows {ROWS_IN_BLOCK} of each block")
    assert torch.isfinite(out.float()).all()
