"""GPU parity: block-sparse prefill against the float64 oracle.

Small configurations are compared on every output element; the large
configurations run at full size in the launch configuration the benchmark
uses and are compared on sampled rows the oracle computes one by one."""
import numpy as np
import pytest

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _mask_for(cfg, scores):
    if cfg.mask_kind == "topk":
        return om.build_mask_topk(scores, cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    return om.build_mask_threshold(scores, cfg.threshold, cfg.dense_last_two_rows, cfg.force_diagonal)


def _run_gpu(qkv, mask, causal):
    q, k, v = (to_gpu_bf16(qkv[n]) for n in ("q", "k", "v"))
    out = bsa.bsattn_fwd(q, k, v, to_gpu(mask), causal)
    return gpu_bf16_to_f64(out)


def _f64(qkv):
    return {n: gen.bf16_bits_to_f64(qkv[n]) for n in ("q", "k", "v")}


@pytest.mark.parametrize("name", ["P0", "P1", "C1", "C2"])
def test_configs_every_element(name):
    cfg = gen.CONFIGS[name]
    inp = gen.prefill_inputs(cfg, 0)
    mask = _mask_for(cfg, inp["scores"])
    say(f"[prefill] {name} B{cfg.B} H{cfg.H} S{cfg.S} D{cfg.D} blocks={int(mask.sum())}")
    got = _run_gpu(inp, mask, cfg.is_causal)
    x = _f64(inp)
    want = oa.prefill(x["q"], x["k"], x["v"], mask, cfg.is_causal)
    check_close(got, want, name)


def _sample_rows(S, nb, rng):
    rows = {0, 1, 63, 64, 65, S // 2, S - 129, S - 65, S - 64, S - 1}
    rows |= set(rng.integers(0, S, size=6).tolist())
    return sorted(r for r in rows if 0 <= r < S)


@pytest.mark.parametrize("name", ["C3", "C4"])
def test_large_configs_sampled_rows(name):
    cfg = gen.CONFIGS[name]
    scores = gen.prefill_scores(cfg, 0)
    mask = _mask_for(cfg, scores)
    qkv = gen.prefill_qkv(cfg, 0)
    say(f"[prefill] {name} full size B{cfg.B} H{cfg.H} S{cfg.S} D{cfg.D} blocks={int(mask.sum())}")
    got = _run_gpu(qkv, mask, cfg.is_causal)
    rng = np.random.default_rng(123)
    heads = [(0, 0), (cfg.B - 1, cfg.H - 1)] + [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H))) for _ in range(2)]
    g_rows, w_rows = [], []
    for b, h in heads:
        rows = _sample_rows(cfg.S, cfg.nb, rng)
        q, k, v = (gen.bf16_bits_to_f64(qkv[n][b, h]) for n in ("q", "k", "v"))
        w_rows.append(oa.prefill_head_rows(q, k, v, mask[b, h], cfg.is_causal, rows))
        g_rows.append(got[b, h, rows])
    check_close(np.concatenate(g_rows), np.concatenate(w_rows), f"{name} sampled rows")
    assert np.isfinite(got).all()


def _random_case(B, H, S, D, seed, density=0.4, causal=True, diag=True):
    rng = np.random.default_rng(seed)
    nb = -(-S // 64)
    mask = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    if diag:
        mask[..., np.arange(nb), np.arange(nb)] = 1
    qkv = {n: gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32)) for n in ("q", "k", "v")}
    return qkv, mask


@pytest.mark.parametrize("S", [1, 63, 64, 65, 200, 383])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_lengths(S, D, causal):
    qkv, mask = _random_case(1, 3, S, D, seed=S * 10 + D + causal, causal=causal)
    say(f"[prefill] ragged S={S} D={D} causal={causal}")
    got = _run_gpu(qkv, mask, causal)
    x = _f64(qkv)
    check_close(got, oa.prefill(x["q"], x["k"], x["v"], mask, causal), f"S{S} D{D} c{causal}")


@pytest.mark.parametrize("B,H", [(2, 4), (1, 8), (3, 5), (2, 16)])
def test_head_counts_and_xcd_mapping(B, H):
    # batch*heads a multiple of 8 takes the XCD-grouped issue order, otherwise the plain one
    qkv, mask = _random_case(B, H, 320, 64, seed=B * 100 + H)
    say(f"[prefill] B{B} H{H} S320")
    got = _run_gpu(qkv, mask, True)
    x = _f64(qkv)
    check_close(got, oa.prefill(x["q"], x["k"], x["v"], mask, True), f"B{B}H{H}")


def test_empty_rows_nonzero_bytes_and_dense():
    qkv, mask = _random_case(1, 4, 256, 64, seed=5, diag=False)
    mask[0, 0] = 0                      # a head with no block at all -> zeros
    mask[0, 1, 2, :] = 0                # one empty query block
    mask[0, 2] = np.tril(np.ones((4, 4), np.uint8)) * 7   # any nonzero byte selects; dense causal
    mask[0, 3] = 1                      # upper blocks are ignored when causal
    say("[prefill] empty rows / nonzero bytes / dense")
    got = _run_gpu(qkv, mask, True)
    x = _f64(qkv)
    want = oa.prefill(x["q"], x["k"], x["v"], mask, True)
    check_close(got, want, "special masks")
    assert (got[0, 0] == 0).all()
    assert (got[0, 1, 128:192] == 0).all()
    # the dense head equals dense causal attention
    import torch
    import torch.nn.functional as F
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x[n][0, 2:3]) for n in ("q", "k", "v")),
                                         is_causal=True).numpy()
    check_close(got[0, 2:3], ref, "dense head vs SDPA")


def test_noncausal_upper_blocks():
    qkv, mask = _random_case(2, 2, 256, 128, seed=9, density=0.5, diag=False)
    mask[..., 0, 3] = 1
    say("[prefill] non-causal upper blocks D128")
    got = _run_gpu(qkv, mask, False)
    x = _f64(qkv)
    check_close(got, oa.prefill(x["q"], x["k"], x["v"], mask, False), "non-causal")


def test_indices_entry_matches_mask_entry_bitwise_and_is_deterministic():
    qkv, mask = _random_case(2, 4, 448, 128, seed=11)
    q, k, v = (to_gpu_bf16(qkv[n]) for n in ("q", "k", "v"))
    m = to_gpu(mask)
    say("[prefill] indices entry / determinism")
    a = bsa.bsattn_fwd(q, k, v, m, True)
    b = bsa.bsattn_fwd(q, k, v, m, True)
    idx, cnt = bsa.bsattn_mask_to_indices(m, True)
    c = bsa.bsattn_fwd_indices(q, k, v, idx, cnt, True)
    import torch
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    # non-causal lists, including out-of-range entries, which are skipped
    idx2, cnt2 = bsa.bsattn_mask_to_indices(m, False)
    idx2[0, 0, 0, -1] = 999
    cnt2[0, 0, 0] = 7
    d = bsa.bsattn_fwd_indices(q, k, v, idx2, cnt2, False)
    x = _f64(qkv)
    want = oa.prefill(x["q"], x["k"], x["v"], mask, False)
    check_close(gpu_bf16_to_f64(d), want, "indices non-causal")


def test_c2_gpu_mask_drives_the_forward_pass():
    # the whole hot path on device: scores -> mask -> forward, vs the oracle end to end
    cfg = gen.CONFIGS["C1"]
    inp = gen.prefill_inputs(cfg, 0)
    say("[prefill] C1 device mask -> forward")
    m = bsa.bsattn_build_mask_topk(to_gpu(inp["scores"]), cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    out = gpu_bf16_to_f64(bsa.bsattn_fwd(q, k, v, m, True))
    mask = om.build_mask_topk(inp["scores"], cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    x = _f64(inp)
    check_close(out, oa.prefill(x["q"], x["k"], x["v"], mask, True), "C1 end to end")


@pytest.mark.parametrize("B,H,D", [(1, 2, 64), (2, 72, 64), (1, 2, 128)])
@pytest.mark.parametrize("dense", [True, False])
def test_rising_scores_take_the_rescale_path(B, H, D, dense):
    """Scores shifted up block by block (one query dimension is a constant,
    the same key dimension grows with the key block), so each later block's
    scores exceed the exponent offset of the blocks before it by more than
    the 2^8 partial-sum margin: the forward's raise-and-redo step runs in the
    pipelined iterations and in the last block.  Within a block the scores
    keep their N(0, 1) spread.  Two heads at D = 64 run with four waves per
    item, 72 heads (1152 items) with two; D = 128."""
    S = 512
    nb = S // 64
    rng = np.random.default_rng(1000 * D + H + dense)
    qf = rng.standard_normal((B, H, S, D), dtype=np.float32)
    kf = rng.standard_normal((B, H, S, D), dtype=np.float32)
    qf[..., D - 1] = 4.0
    kf[..., D - 1] = np.repeat(np.arange(nb, dtype=np.float32) * (150.0 if D == 64 else 250.0), 64)
    q, k = gen.f32_to_bf16_bits(qf), gen.f32_to_bf16_bits(kf)
    # Rows early in a diagonal block attend to one or two keys, so their
    # outputs are single values of V: V ~ N(0, 1/16) keeps those near 1, where
    # the bfloat16 rounding of the output itself stays well inside the
    # tolerance (at |o| >= 4 a half unit in the last place is 0.0156).
    v = gen.f32_to_bf16_bits(0.25 * rng.standard_normal((B, H, S, D), dtype=np.float32))
    if dense:
        mask = np.ones((B, H, nb, nb), np.uint8)
    else:
        mask = (rng.random((B, H, nb, nb)) < 0.6).astype(np.uint8)
        mask[..., np.arange(nb), np.arange(nb)] = 1
    x = {n: gen.bf16_bits_to_f64(a) for n, a in (("q", q), ("k", k), ("v", v))}
    # the data does what the test is for: in every row with two or more
    # blocks, each block's maximum exceeds the previous block's by more than
    # 8 / c (the margin of the lazy exponent offset)
    c = np.log2(np.e) / np.sqrt(D)
    s = (x["q"][0, 0] @ x["k"][0, 0].T) / np.sqrt(D)
    for r in range(64, S):
        i = r // 64
        sel = [j for j in range(i + 1) if mask[0, 0, i, j]]
        mx = [s[r, 64 * j:min(64 * j + 64, r + 1)].max() for j in sel]
        assert all((b - a) * c > 10 for a, b in zip(mx, mx[1:])), (r, mx)
    say(f"[prefill] rising scores B{B} H{H} D{D} dense={dense}")
    got = _run_gpu({"q": q, "k": k, "v": v}, mask, True)
    want = oa.prefill(x["q"], x["k"], x["v"], mask, True)
    check_close(got, want, f"rising scores B{B} H{H} D{D}")
    if dense:
        # the fused form (row selection in the forward's prologue) runs the
        # same redo: top-k with k = nb keeps every causal block
        say(f"[prefill] rising scores, fused top-k, B{B} H{H} D{D}")
        fused = bsa.bsattn_fwd_topk(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v),
                                    to_gpu(np.zeros((B, H, nb, nb), np.float32)), nb)
        check_close(gpu_bf16_to_f64(fused), want, f"rising scores fused B{B} H{H} D{D}")


def _long_row_mask(H, nb, seed, heavy=True):
    rng = np.random.default_rng(seed)
    mask = (rng.random((1, H, nb, nb)) < 0.05).astype(np.uint8)
    mask[..., np.arange(nb), np.arange(nb)] = 1
    if heavy:
        for h in range(H - 1):          # the last head keeps light rows: its helpers have nothing to do
            mask[0, h, 128, :129] = 1   # 129 blocks: split 64 / 65
            mask[0, h, 129, :130] = 1   # 130 blocks: split 65 / 65
            if h % 2:
                mask[0, h, 129, [3, 77]] = 0   # exactly 128 blocks: not split
    return mask


@pytest.mark.parametrize("S", [8320, 8300])
@pytest.mark.parametrize("H,D", [(8, 64), (4, 64), (8, 128)])
def test_long_rows_split_in_two(S, H, D):
    """Causal query blocks with more than 128 key blocks run as two halves and a
    merge; one workspace serves a call with long rows, then one without (the
    split flags of the first must not leak into the second)."""
    import torch
    nb = -(-S // 64)
    need = bsa.bsattn_fwd_workspace_bytes(1, H, S, D)
    assert need > 0
    rng = np.random.default_rng(S + H + D)
    qkv = {n: gen.f32_to_bf16_bits(rng.standard_normal((1, H, S, D), dtype=np.float32)) for n in ("q", "k", "v")}
    q, k, v = (to_gpu_bf16(qkv[n]) for n in ("q", "k", "v"))
    x = _f64(qkv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rows = sorted(set(range(128 * 64, S)) | {0, 64 * 127, 64 * 127 + 63, S // 2})
    for heavy in (True, False):
        mask = _long_row_mask(H, nb, seed=S * 7 + D, heavy=heavy)
        say(f"[prefill] long rows S={S} H={H} D={D} heavy={heavy} blocks={int(mask.sum())}")
        got = gpu_bf16_to_f64(bsa.bsattn_fwd(q, k, v, to_gpu(mask), True, workspace=ws))
        want = np.stack([oa.prefill_head_rows(x["q"][0, h], x["k"][0, h], x["v"][0, h], mask[0, h], True, rows)
                         for h in range(H)])
        check_close(got[0][:, rows], want, f"S{S} H{H} D{D} heavy={heavy}")


def test_long_rows_noncausal_run_whole():
    """Non-causal calls never split (every row may see every block): no
    workspace is passed, and rows of 130 blocks run whole."""
    S, H, D = 8300, 4, 64
    nb = -(-S // 64)
    assert bsa.bsattn_fwd_workspace_bytes(1, H, S, D) > 0
    rng = np.random.default_rng(77)
    qkv = {n: gen.f32_to_bf16_bits(rng.standard_normal((1, H, S, D), dtype=np.float32)) for n in ("q", "k", "v")}
    mask = (rng.random((1, H, nb, nb)) < 0.05).astype(np.uint8)
    mask[0, :, 127:] = 1                # dense rows, past the diagonal too
    say(f"[prefill] long rows non-causal S={S} H={H} D={D} blocks={int(mask.sum())}")
    got = _run_gpu(qkv, mask, False)
    x = _f64(qkv)
    rows = sorted(set(range(127 * 64, S)) | {0, 1, S // 2})
    want = np.stack([oa.prefill_head_rows(x["q"][0, h], x["k"][0, h], x["v"][0, h], mask[0, h], False, rows)
                     for h in range(H)])
    check_close(got[0][:, rows], want, "long rows non-causal")
