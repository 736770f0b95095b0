"""GPU parity: the XAttention estimator (block sums and cumulative selection)
against the float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import xattn as ox
from tests.gpu_util import parallel_map, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

# Block sums: float32 logits from bf16 products summed in fp32, exp2/log2 in
# float32; relative error of a weight stays far below 1e-5 at these sizes.
SUM_RTOL, SUM_ATOL = 1e-4, 1e-6


def _qk(B, H, Sq, Sk, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sq, D), dtype=np.float32) * scale)
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32) * scale)
    return q, k


def _estimate_rows(B, H, nbq, nbk, seed, grid):
    """Nonnegative rows shaped like an estimate: zero after the diagonal."""
    rng = np.random.default_rng(seed)
    x = rng.random((B, H, nbq, nbk)).astype(np.float32) ** 3
    if grid:
        x = (np.round(x * 64) / 64).astype(np.float32)   # many ties and exact zeros
    past = nbk - nbq
    for i in range(nbq):
        x[..., i, i + past + 1:] = 0
    return x


@pytest.mark.parametrize("nbq,nbk", [(1, 1), (5, 5), (64, 64), (37, 100), (256, 256), (8, 1024)])
@pytest.mark.parametrize("grid", [False, True])
def test_cumulative_selection_bit_exact(nbq, nbk, grid):
    B, H = 2, 3
    x = _estimate_rows(B, H, nbq, nbk, nbq * 7 + nbk + grid, grid)
    xs = to_gpu(x)
    for thr in (0.0, 0.5, 0.9, 0.97, 1.0):
        for sink, diag, causal in ((True, True, True), (False, True, True), (True, False, False),
                                   (False, False, True)):
            say(f"[xattn-select] nbq={nbq} nbk={nbk} grid={grid} thr={thr} sink={sink} diag={diag} causal={causal}")
            got = bsa.bsattn_build_mask_cumulative(xs, thr, sink, diag, causal).cpu().numpy()
            want = ox.find_blocks(x, thr, sink, diag, causal)
            np.testing.assert_array_equal(got, want)


def test_cumulative_selection_general_values():
    # negative weights, signed zeros and dense future columns: still the rule, bit for bit
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 4, 20, 33)).astype(np.float32)
    x[0, 0, :, :5] = 0.0
    x[0, 1, :, :5] = -0.0
    for thr in (0.3, 0.9):
        say(f"[xattn-select] general values thr={thr}")
        got = bsa.bsattn_build_mask_cumulative(to_gpu(x), thr, True, True, False).cpu().numpy()
        np.testing.assert_array_equal(got, ox.find_blocks(x, thr, True, True, False))


CASES = [
    # B, H, Sq, Sk, D, stride, causal
    (1, 2, 256, 256, 64, 8, True),
    (2, 1, 200, 200, 64, 8, True),       # ragged: the last block has 8 tokens
    (1, 2, 2048, 2048, 128, 8, True),    # 2 x 2 reshaped tiles
    (1, 1, 1024, 1024, 128, 4, True),
    (1, 1, 2560, 2560, 64, 16, True),
    (1, 2, 64, 64, 64, 16, True),        # one block
    (1, 2, 512, 1536, 128, 8, True),     # a chunk: the last 512 of 1536 positions
    (1, 1, 448, 1088, 64, 4, False),
    (1, 2, 640, 640, 128, 16, False),
]


def _oracle_sums(q, k, stride, norm, causal):
    f = gen.bf16_bits_to_f64
    return ox.block_sums(f(q), f(k), stride, norm, causal)


@pytest.mark.parametrize("B,H,Sq,Sk,D,stride,causal", CASES)
def test_block_sums(B, H, Sq, Sk, D, stride, causal):
    q, k = _qk(B, H, Sq, Sk, D, Sq + 3 * Sk + D + stride)
    say(f"[xattn-sums] B={B} H={H} Sq={Sq} Sk={Sk} D={D} stride={stride} causal={causal}")
    got = bsa.bsattn_xattn_block_sums(to_gpu_bf16(q), to_gpu_bf16(k), stride, 1.0, causal)
    got = got.cpu().numpy().astype(np.float64)
    want = _oracle_sums(q, k, stride, 1.0, causal)
    err = np.abs(got - want)
    say(f"  max abs {err.max():.3e}, max rel {(err / np.maximum(want, 1e-30)).max():.3e}")
    np.testing.assert_allclose(got, want, rtol=SUM_RTOL, atol=SUM_ATOL)
    # each query block's row adds up to its number of reshaped rows
    rows = Sq // stride
    b = 64 // stride
    tot = [min(b, rows - i * b) for i in range(got.shape[2])]
    np.testing.assert_allclose(got.sum(axis=-1), np.broadcast_to(tot, got.shape[:3]), rtol=1e-5)


def test_norm_and_sharp_logits():
    # norm 0.5 and inputs scaled by 3: sharp rows where one key dominates
    q, k = _qk(1, 2, 512, 512, 64, 11, scale=3.0)
    for norm in (0.5, 2.0):
        say(f"[xattn-sums] norm={norm}")
        got = bsa.bsattn_xattn_block_sums(to_gpu_bf16(q), to_gpu_bf16(k), 8, norm, True)
        np.testing.assert_allclose(got.cpu().numpy(), _oracle_sums(q, k, 8, norm, True),
                                   rtol=SUM_RTOL, atol=SUM_ATOL)


def _check_valid_selection(mask, sums, thr, sink, diag, causal, tol):
    """The GPU selection, judged on the oracle's block sums: forced columns kept,
    nothing after the diagonal, and the kept unforced columns a top-weighted set
    whose weight reaches thr * total while dropping its lightest member would
    not (each up to tol, the block-sum tolerance summed over a row)."""
    nbq, nbk = sums.shape[-2:]
    past = nbk - nbq
    for idx in np.ndindex(*sums.shape[:-1]):
        i = idx[-1]
        d = i + past
        m = mask[idx].astype(bool)
        w = sums[idx]
        forced = {c for c, on in ((0, sink), (d, diag)) if on}
        for c in forced:
            assert m[c], (idx, c)
        if causal:
            assert not m[d + 1:].any(), idx
        free = np.array([c for c in range(nbk) if c not in forced and (not causal or c <= d)], int)
        if free.size == 0:
            continue
        kept, dropped = free[m[free]], free[~m[free]]
        req = thr * w.sum()
        kw = w[kept].sum()
        if dropped.size and kept.size:
            assert w[kept].min() >= w[dropped].max() - tol, idx
        if dropped.size and w[dropped].max() > tol:
            assert kw >= req - tol, (idx, kw, req)
        if kept.size:
            assert kw - w[kept].min() < req + tol, (idx, kw, req)


@pytest.mark.parametrize("B,H,Sq,Sk,D,stride,causal", CASES[:7])
def test_estimate_mask(B, H, Sq, Sk, D, stride, causal):
    q, k = _qk(B, H, Sq, Sk, D, 5 * Sq + Sk + D + stride)
    want_sums = _oracle_sums(q, k, stride, 1.0, causal)
    for thr, sink, diag in ((0.9, True, True), (0.6, False, True), (0.95, True, False)):
        say(f"[xattn-estimate] B={B} H={H} Sq={Sq} Sk={Sk} D={D} s={stride} thr={thr} sink={sink} diag={diag}")
        mask, sums = bsa.bsattn_xattn_estimate(to_gpu_bf16(q), to_gpu_bf16(k), stride, 1.0, thr, sink,
                                               diag, causal, write_sums=True)
        mask = mask.cpu().numpy()
        sums_g = sums.cpu().numpy()
        np.testing.assert_allclose(sums_g, want_sums, rtol=SUM_RTOL, atol=SUM_ATOL)
        tol = sums_g.shape[-1] * (SUM_ATOL + SUM_RTOL * 64 / stride)
        _check_valid_selection(mask, want_sums, thr, sink, diag, causal, tol)
        want = ox.find_blocks(want_sums.astype(np.float32), thr, sink, diag, causal)
        same = (mask == want).all(axis=-1).mean()
        say(f"  rows identical to the oracle's selection: {100 * same:.2f}%")
        # the estimate without the block-sums output gives the same mask
        m2 = bsa.bsattn_xattn_estimate(to_gpu_bf16(q), to_gpu_bf16(k), stride, 1.0, thr, sink, diag, causal)
        np.testing.assert_array_equal(m2.cpu().numpy(), mask)


def test_full_size_every_head():
    """The 16384-token, 32-head, D 128 prefill shape at stride 8: every head's
    block sums against the oracle, and every head's selection valid for them."""
    cfg = gen.CONFIGS["C3"]
    qkv = gen.prefill_qkv(cfg, 0)
    q, k = to_gpu_bf16(qkv["q"]), to_gpu_bf16(qkv["k"])
    say("[xattn-estimate] full size B1 H32 S16384 D128 stride 8")
    mask, sums = bsa.bsattn_xattn_estimate(q, k, 8, 1.0, 0.9, True, True, True, write_sums=True)
    sums = sums.cpu().numpy()
    mask = mask.cpu().numpy()
    f = gen.bf16_bits_to_f64
    say(f"  oracle block sums on {cfg.H} heads")
    wants = parallel_map(lambda h: ox.block_sums(f(qkv["q"][:, h:h + 1]), f(qkv["k"][:, h:h + 1]),
                                                 8, 1.0, True), range(cfg.H))
    tol = 256 * (SUM_ATOL + SUM_RTOL * 8)
    for h, want in enumerate(wants):
        np.testing.assert_allclose(sums[:, h:h + 1], want, rtol=SUM_RTOL, atol=SUM_ATOL)
        _check_valid_selection(mask[:, h:h + 1], want, 0.9, True, True, True, tol)
    # every head: rows add up to 8 reshaped rows, nothing after the diagonal
    np.testing.assert_allclose(sums.sum(axis=-1), 8.0, rtol=1e-5)
    assert not np.triu(mask, 1).any()


def test_deterministic():
    q, k = _qk(1, 4, 1024, 1024, 128, 21)
    qg, kg = to_gpu_bf16(q), to_gpu_bf16(k)
    say("[xattn-estimate] determinism")
    m1, s1 = bsa.bsattn_xattn_estimate(qg, kg, 8, 1.0, 0.9, True, True, True, write_sums=True)
    m2, s2 = bsa.bsattn_xattn_estimate(qg, kg, 8, 1.0, 0.9, True, True, True, write_sums=True)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(m1, m2)
