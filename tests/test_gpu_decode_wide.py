"""GPU parity: sparse GQA decode with query-head groups beyond 16 (up to the
guide's block_H of 64, §6.1) and a value head dim different from the key
head dim (the guide's dim_v, §9.2), in the index, mask and paged forms,
against the float64 oracle on every output element."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

f64 = gen.bf16_bits_to_f64


def _case(seed, D, Dv, G, Hkv=2, lens=(1, 63, 64, 65, 200, 1000, 3000)):
    rng = np.random.default_rng(seed)
    lens = np.array(lens)
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    ms = 12
    idx = np.full((B, Hkv, ms), -1, np.int32)
    for b, L in enumerate(lens):
        nbb = -(-int(L) // 64)
        for h in range(Hkv):
            n = int(rng.integers(1, min(nbb, ms - 2) + 1))
            row = list(rng.choice(nbb, size=n, replace=False)) + [nbb + 1, -3]
            rng.shuffle(row)
            idx[b, h, :len(row)] = row
    nbk = max(-(-int(x) // 64) for x in lens)
    bm = np.zeros((B, Hkv, nbk), np.uint8)
    for b in range(B):
        for h in range(Hkv):
            s = idx[b, h]
            bm[b, h, s[(s >= 0) & (s < nbk)]] = 1
    return {"lens": lens, "cu_seqlens_k": cu, "block_indices": idx, "block_mask": bm,
            "q": gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv * G, D), dtype=np.float32)),
            "k": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32)),
            "v": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, Dv), dtype=np.float32))}


SHAPES = [(128, 128, 32), (128, 128, 64), (64, 128, 4), (128, 64, 8), (64, 64, 48), (128, 64, 64),
          (64, 128, 20)]


@pytest.mark.parametrize("D,Dv,G", SHAPES)
def test_index_and_mask_forms(D, Dv, G):
    d = _case(D * 7 + Dv + G, D, Dv, G)
    want = oa.decode_gqa(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_seqlens_k"], d["block_indices"])
    want_m = oa.decode_gqa_mask(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_seqlens_k"], d["block_mask"])
    np.testing.assert_allclose(want, want_m, rtol=1e-12, atol=1e-12)   # the same selection
    q, k, v = (to_gpu_bf16(d[n]) for n in ("q", "k", "v"))
    cu, idx, bm = to_gpu(d["cu_seqlens_k"]), to_gpu(d["block_indices"]), to_gpu(d["block_mask"])
    for ns in (0, 1, 3):
        say(f"[decode-wide] D={D} Dv={Dv} G={G} ns={ns}")
        o = bsa.bsattn_decode_gqa(q, k, v, cu, idx, num_splits=ns)
        assert tuple(o.shape) == (len(d["lens"]), 2 * G, Dv)
        check_close(gpu_bf16_to_f64(o), want, f"index D{D} Dv{Dv} G{G} ns{ns}")
        om = bsa.bsattn_decode_gqa_mask(q, k, v, cu, bm, num_splits=ns)
        check_close(gpu_bf16_to_f64(om), want, f"mask D{D} Dv{Dv} G{G} ns{ns}")
        if ns:
            na = bsa.bsattn_decode_gqa_noalloc(q, k, v, cu, idx, num_splits=ns)
            assert torch.equal(na.view(torch.int16), o.view(torch.int16))


@pytest.mark.parametrize("D,Dv,G", [(128, 128, 64), (64, 128, 32), (128, 64, 16)])
def test_paged_form(D, Dv, G):
    rng = np.random.default_rng(D + Dv + G)
    lens = np.array([100, 1500, 700])
    B, Hkv, page = len(lens), 2, 128
    per = [-(-int(x) // page) for x in lens]
    num_pages = sum(per) + 3
    perm = rng.permutation(num_pages)
    kc = gen.f32_to_bf16_bits(rng.standard_normal((num_pages, page, Hkv, D), dtype=np.float32))
    vc = gen.f32_to_bf16_bits(rng.standard_normal((num_pages, page, Hkv, Dv), dtype=np.float32))
    table = np.full((B, max(per)), -1, np.int32)
    p = 0
    for b in range(B):
        for lp in range(per[b]):
            table[b, lp] = perm[p]
            p += 1
    idx = np.full((B, Hkv, 8), -1, np.int32)
    for b, L in enumerate(lens):
        nbb = -(-int(L) // 64)
        for h in range(Hkv):
            n = int(rng.integers(1, min(nbb, 8) + 1))
            idx[b, h, :n] = rng.choice(nbb, size=n, replace=False)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv * G, D), dtype=np.float32))
    want = oa.decode_gqa_paged(f64(q), f64(kc), f64(vc), lens.astype(np.int32), table, idx)
    for ns in (1, 4):
        say(f"[decode-wide] paged D={D} Dv={Dv} G={G} ns={ns}")
        o = bsa.bsattn_decode_gqa_paged(to_gpu_bf16(q), to_gpu_bf16(kc), to_gpu_bf16(vc),
                                        to_gpu(lens.astype(np.int32)), to_gpu(table), to_gpu(idx),
                                        num_splits=ns)
        check_close(gpu_bf16_to_f64(o), want, f"paged D{D} Dv{Dv} G{G} ns{ns}")


def test_group_of_64_at_workload_size():
    """B8, 64 query heads over one KV head, D 128, KV lengths U[4096, 32768], up
    to 64 selected blocks: the group-64 form at the decode workload's scale."""
    cfg = gen.DecodeConfig("g64", 8, 64, 1, 128, 4096, 32768)
    d = gen.decode_inputs(cfg, 3)
    want = oa.decode_gqa(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["cu_seqlens_k"], d["block_indices"])
    q, k, v = (to_gpu_bf16(d[n]) for n in ("q", "k", "v"))
    for ns in (0, 2):
        say(f"[decode-wide] B8 Hq64 Hkv1 D128 ns={ns}")
        o = bsa.bsattn_decode_gqa(q, k, v, to_gpu(d["cu_seqlens_k"]), to_gpu(d["block_indices"]),
                                  num_splits=ns)
        check_close(gpu_bf16_to_f64(o), want, f"group 64 ns{ns}")
