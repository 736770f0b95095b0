"""GPU parity: split-KV sparse GQA decode against the float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _gpu(inp, ns, cu=None):
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    cu_t = to_gpu(inp["cu_seqlens_k"] if cu is None else cu)
    out = bsa.bsattn_decode_gqa(q, k, v, cu_t, to_gpu(inp["block_indices"]), num_splits=ns)
    return out


def _oracle(inp):
    x = {n: gen.bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v")}
    return oa.decode_gqa(x["q"], x["k"], x["v"], inp["cu_seqlens_k"], inp["block_indices"])


@pytest.mark.parametrize("name", ["P2", "C5"])
def test_configs(name):
    cfg = gen.CONFIGS[name]
    inp = gen.decode_inputs(cfg, 0)
    want = _oracle(inp)
    default = bsa.bsattn_decode_default_splits(cfg.B, cfg.Hq, cfg.Hkv, cfg.max_selected_blocks, cfg.D)
    say(f"[decode] {name} total_k={int(inp['cu_seqlens_k'][-1])} default splits={default}")
    outs = []
    for ns in (0, 1, 3, cfg.max_selected_blocks):
        say(f"[decode] {name} num_splits={ns}")
        o = _gpu(inp, ns)
        outs.append(gpu_bf16_to_f64(o))
        check_close(outs[-1], want, f"{name} ns={ns}")
    # split invariance beyond the oracle comparison
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-2


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_ragged_small(D, G):
    rng = np.random.default_rng(D + G)
    lens = np.array([1, 63, 64, 65, 200, 1000])
    B, Hkv = len(lens), 2
    Hq = Hkv * G
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    ms = 9
    idx = np.full((B, Hkv, ms), -1, np.int32)
    for b, L in enumerate(lens):
        nbb = -(-int(L) // 64)
        for h in range(Hkv):
            n = int(rng.integers(1, min(nbb, ms - 2) + 1))
            sel = rng.choice(nbb, size=n, replace=False)
            row = list(sel) + [nbb + 3, -5]      # out-of-range entries are skipped
            rng.shuffle(row)                      # order does not matter
            idx[b, h, :len(row)] = row
    inp = {"lens": lens, "cu_seqlens_k": cu, "block_indices": idx,
           "q": gen.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32)),
           "k": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32)),
           "v": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))}
    want = _oracle(inp)
    for ns in (1, 2, ms):
        say(f"[decode] ragged D={D} G={G} ns={ns}")
        check_close(gpu_bf16_to_f64(_gpu(inp, ns)), want, f"D{D} G{G} ns{ns}")


def test_all_padding_and_malformed_lengths():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, D = 3, 8, 2, 128
    lens = np.array([128, 100, 64])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    idx = np.full((B, Hkv, 4), -1, np.int32)
    idx[0, :, :2] = [[1, 0], [0, -1]]
    idx[2, :, 0] = 0
    inp = {"cu_seqlens_k": cu, "block_indices": idx,
           "q": gen.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32)),
           "k": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32)),
           "v": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))}
    want = _oracle(inp)
    say("[decode] all-padding batch")
    got = gpu_bf16_to_f64(_gpu(inp, 2))
    check_close(got, want, "padding")
    assert (got[1] == 0).all()
    # a sequence whose range runs past total_k is read as empty
    bad = cu.copy()
    bad[3] = T + 500
    say("[decode] malformed cu_seqlens")
    got2 = gpu_bf16_to_f64(_gpu(inp, 2, cu=bad))
    assert (got2[2] == 0).all()
    np.testing.assert_array_equal(got2[:2], got[:2])


def test_deterministic():
    cfg = gen.CONFIGS["P2"]
    inp = gen.decode_inputs(cfg, 1)
    say("[decode] determinism")
    a = _gpu(inp, 4)
    b = _gpu(inp, 4)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_needs_no_clearing():
    """Workspace contents left by anything (garbage, earlier calls, another
    split count) must not change the result."""
    cfg = gen.CONFIGS["P2"]
    inp = gen.decode_inputs(cfg, 2)
    want = _oracle(inp)
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    cu, idx = to_gpu(inp["cu_seqlens_k"]), to_gpu(inp["block_indices"])
    big = bsa.bsattn_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.D, cfg.max_selected_blocks)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    outs = []
    for fill, ns in ((0xFF, 4), (None, 4), (0x00, 4), (None, 7), (None, 4), (0x5A, 2)):
        if fill is not None:
            ws.fill_(fill)
        say(f"[decode] workspace fill={fill} ns={ns}")
        o = bsa.bsattn_decode_gqa(q, k, v, cu, idx, num_splits=ns, workspace=ws)
        outs.append(gpu_bf16_to_f64(o))
        check_close(outs[-1], want, f"ws fill={fill} ns={ns}")
    # the same split count gives bit-identical results whatever the workspace held
    for i in (1, 2, 4):
        np.testing.assert_array_equal(outs[i], outs[0])
