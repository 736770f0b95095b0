"""Guard regions around every buffer the library writes.

Each output, list and workspace is the middle of a larger allocation whose
head and tail (4 KiB each) hold a known byte pattern; after the call the
pattern must be intact, so a write past either end of a buffer (a ragged
tail row, a split-row half, a padded list, a paged table lookup) cannot go
unseen even where the values inside the buffer are right.  Results inside
the buffers are compared with the oracle as elsewhere.  Shapes: ragged
sequence lengths, chunks of queries, causal rows long enough to split,
ragged and paged decode, the estimator.  (The block-sparse guide's §6.2
handles the ends of variable-length sequences by bounds; these tests check
that the library's own bounds hold.)"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from oracle import xattn as ox
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

PAD = 4096
PATTERN = 0xA5


class Guarded:
    """A device tensor of `shape` and `dtype` (initialised to the pattern
    bytes) with PAD guard bytes before and after it."""

    def __init__(self, shape, dtype):
        itemsize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * itemsize
        self.buf = torch.full((n + 2 * PAD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + n].view(dtype).view(tuple(shape))
        self.n = n

    def check(self, what):
        torch.cuda.synchronize()
        head = self.buf[:PAD].cpu().numpy()
        tail = self.buf[PAD + self.n:].cpu().numpy()
        assert (head == PATTERN).all(), f"{what}: write before the buffer"
        assert (tail == PATTERN).all(), f"{what}: write after the buffer"


def _qkv(rng, B, H, S, D):
    return {n: gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D), dtype=np.float32))
            for n in ("q", "k", "v")}


def _f64(d):
    return {n: gen.bf16_bits_to_f64(d[n]) for n in ("q", "k", "v")}


@pytest.mark.parametrize("S", [1, 63, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged(S, D, causal):
    rng = np.random.default_rng(S * 7 + D + causal)
    B, H = 1, 3
    nb = -(-S // 64)
    x = _qkv(rng, B, H, S, D)
    scores = rng.standard_normal((B, H, nb, nb), dtype=np.float32)
    q, k, v = (to_gpu_bf16(x[n]) for n in ("q", "k", "v"))
    topk = max(1, nb // 2)
    say(f"[guards] prefill S={S} D={D} causal={causal}")
    mg = Guarded((B, H, nb, nb), torch.uint8)
    bsa.bsattn_build_mask_topk(to_gpu(scores), topk, True, True, out=mg.t)
    mg.check("top-k mask")
    mask = om.build_mask_topk(scores, topk, True, True)
    np.testing.assert_array_equal(mg.t.cpu().numpy(), mask)
    tg = Guarded((B, H, nb, nb), torch.uint8)
    bsa.bsattn_build_mask_threshold(to_gpu(scores), 0.2, True, True, out=tg.t)
    tg.check("threshold mask")
    ig, cg = Guarded((B, H, nb, nb), torch.int32), Guarded((B, H, nb), torch.int32)
    bsa.bsattn_mask_to_indices(mg.t, causal, idx=ig.t, cnt=cg.t)
    ig.check("compaction idx")
    cg.check("compaction cnt")
    want = oa.prefill(*(_f64(x)[n] for n in ("q", "k", "v")), mask, causal)
    for form in ("mask", "indices", "fused"):
        og = Guarded((B, H, S, D), torch.bfloat16)
        if form == "mask":
            bsa.bsattn_fwd(q, k, v, mg.t, causal, out=og.t)
        elif form == "indices":
            bsa.bsattn_fwd_indices(q, k, v, ig.t, cg.t, causal, out=og.t)
        else:
            fm = Guarded((B, H, nb, nb), torch.uint8)
            bsa.bsattn_fwd_topk(q, k, v, to_gpu(scores), topk, True, True, causal, out=og.t,
                                mask_out=fm.t)
            fm.check("fused mask output")
            np.testing.assert_array_equal(fm.t.cpu().numpy(), mask)
        og.check(f"forward output ({form})")
        check_close(gpu_bf16_to_f64(og.t), want, f"S{S} D{D} {form}")


@pytest.mark.parametrize("Sq,Sk", [(1, 70), (100, 1000), (64, 129), (200, 200)])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_chunk(Sq, Sk, D):
    rng = np.random.default_rng(Sq + Sk + D)
    B, H = 2, 2
    nbq, nbk = -(-Sq // 64), -(-Sk // 64)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sq, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    mask = (rng.random((B, H, nbq, nbk)) < 0.5).astype(np.uint8)
    say(f"[guards] chunk Sq={Sq} Sk={Sk} D={D}")
    og = Guarded((B, H, Sq, D), torch.bfloat16)
    bsa.bsattn_fwd_chunk(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), to_gpu(mask), True, out=og.t)
    og.check("chunk output")
    f = gen.bf16_bits_to_f64
    check_close(gpu_bf16_to_f64(og.t), oa.prefill(f(q), f(k), f(v), mask, True), f"chunk {Sq}/{Sk}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_split_rows(D):
    """Causal rows past 128 key blocks: the item and its helper write halves
    to the workspace and the merge writes the output."""
    rng = np.random.default_rng(D)
    B, H, S = 1, 2, 8300
    nb = -(-S // 64)
    x = _qkv(rng, B, H, S, D)
    mask = (rng.random((B, H, nb, nb)) < 0.2).astype(np.uint8)
    mask[..., nb - 3:, :] = 1          # three long rows per head: two split, one does not
    mask[..., nb - 1, 5] = 0
    mask[..., np.arange(nb), np.arange(nb)] = 1
    need = bsa.bsattn_fwd_workspace_bytes(B, H, S, D)
    assert need > 0
    say(f"[guards] split rows S={S} D={D} workspace={need}")
    og, wg = Guarded((B, H, S, D), torch.bfloat16), Guarded((need,), torch.uint8)
    q, k, v = (to_gpu_bf16(x[n]) for n in ("q", "k", "v"))
    bsa.bsattn_fwd(q, k, v, to_gpu(mask), True, out=og.t, workspace=wg.t)
    og.check("split-row output")
    wg.check("split-row workspace")
    rows = list(range(64 * (nb - 3), S)) + [0, 63, 4000, 8191]
    f = _f64(x)
    want = np.stack([oa.prefill_head_rows(f["q"][0, h], f["k"][0, h], f["v"][0, h], mask[0, h], True, rows)
                     for h in range(H)])
    got = gpu_bf16_to_f64(og.t)[0][:, rows]
    check_close(got, want, f"split rows D{D}")


def _ragged_decode(rng, D, G):
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
            row = list(rng.choice(nbb, size=n, replace=False)) + [nbb + 3, -5]
            idx[b, h, :len(row)] = row
    return {"lens": lens, "cu_seqlens_k": cu, "block_indices": idx,
            "q": gen.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32)),
            "k": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32)),
            "v": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_decode_ragged(D, G):
    rng = np.random.default_rng(100 + D + G)
    inp = _ragged_decode(rng, D, G)
    B, Hq, _ = inp["q"].shape
    Hkv = inp["k"].shape[1]
    ms = inp["block_indices"].shape[2]
    want = oa.decode_gqa(*(gen.bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v")),
                         inp["cu_seqlens_k"], inp["block_indices"])
    nbk = max(-(-int(x) // 64) for x in inp["lens"])
    bm = np.zeros((B, Hkv, nbk), np.uint8)
    for b in range(B):
        for h in range(Hkv):
            sel = inp["block_indices"][b, h]
            sel = sel[(sel >= 0) & (sel < nbk)]
            bm[b, h, sel] = 1
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    cu = to_gpu(inp["cu_seqlens_k"])
    for ns in (1, 3):
        for form in ("indices", "mask"):
            say(f"[guards] decode D={D} G={G} ns={ns} {form}")
            need = bsa.bsattn_decode_workspace_bytes(B, Hq, D, ns)
            og = Guarded((B, Hq, D), torch.bfloat16)
            wg = Guarded((max(need, 1),), torch.uint8)
            if form == "indices":
                bsa.bsattn_decode_gqa(q, k, v, cu, to_gpu(inp["block_indices"]), num_splits=ns,
                                      out=og.t, workspace=wg.t)
            else:
                bsa.bsattn_decode_gqa_mask(q, k, v, cu, to_gpu(bm), num_splits=ns, out=og.t,
                                           workspace=wg.t)
            og.check(f"decode output ({form})")
            wg.check(f"decode workspace ({form})")
            check_close(gpu_bf16_to_f64(og.t), want, f"decode D{D} G{G} ns{ns} {form}")


@pytest.mark.parametrize("page_size", [64, 256])
def test_decode_paged(page_size):
    base = gen.decode_inputs(gen.DecodeConfig("g", 3, 16, 4, 128, 100, 3000), 7)
    d = gen.decode_paged_inputs(gen.DecodeConfig("g", 3, 16, 4, 128, 100, 3000), 7,
                                page_size=page_size, base=base)
    B, Hq, D = d["q"].shape
    ns = 4
    need = bsa.bsattn_decode_workspace_bytes(B, Hq, D, ns)
    og, wg = Guarded((B, Hq, D), torch.bfloat16), Guarded((need,), torch.uint8)
    say(f"[guards] paged decode page={page_size}")
    bsa.bsattn_decode_gqa_paged(to_gpu_bf16(d["q"]), to_gpu_bf16(d["k_cache"]), to_gpu_bf16(d["v_cache"]),
                                to_gpu(d["cache_seqlens"]), to_gpu(d["block_table"]),
                                to_gpu(d["block_indices"]), num_splits=ns, out=og.t, workspace=wg.t)
    og.check("paged decode output")
    wg.check("paged decode workspace")
    f = gen.bf16_bits_to_f64
    want = oa.decode_gqa_paged(f(d["q"]), f(d["k_cache"]), f(d["v_cache"]), d["cache_seqlens"],
                               d["block_table"], d["block_indices"])
    check_close(gpu_bf16_to_f64(og.t), want, f"paged {page_size}")


@pytest.mark.parametrize("Sq,Sk,stride", [(1000, 1000, 8), (320, 960, 4), (512, 2048, 16)])
def test_xattn(Sq, Sk, stride):
    rng = np.random.default_rng(Sq + Sk + stride)
    B, H, D = 1, 3, 64
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sq, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    nbq, nbk = -(-Sq // 64), -(-Sk // 64)
    need = bsa.bsattn_xattn_workspace_bytes(B, H, Sq, Sk, stride)
    sg, mg = Guarded((B, H, nbq, nbk), torch.float32), Guarded((B, H, nbq, nbk), torch.uint8)
    wg = Guarded((need,), torch.uint8)
    say(f"[guards] xattn Sq={Sq} Sk={Sk} s={stride}")
    bsa.bsattn_xattn_estimate(to_gpu_bf16(q), to_gpu_bf16(k), stride, 1.0, 0.9, True, True, True,
                              block_sums=sg.t, out=mg.t, workspace=wg.t)
    sg.check("estimator block sums")
    mg.check("estimator mask")
    wg.check("estimator workspace")
    f = gen.bf16_bits_to_f64
    want = ox.block_sums(f(q), f(k), stride, 1.0, True)
    np.testing.assert_allclose(sg.t.cpu().numpy(), want, rtol=1e-4, atol=1e-6)
    assert math.isfinite(float(sg.t.sum()))
