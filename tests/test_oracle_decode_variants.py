"""Pins for the mask-form and paged-KV decode oracles (CPU only).

Both are checked against torch's scaled_dot_product_attention in float64 (a
library routine) on a token-level mask that the test builds on its own
(np.repeat of the block selection), against closed forms, and, for the paged
layout, on caches the test scatters into shuffled pages itself."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as oa

BLOCK = 64


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa_one(qv, kk, vv, allowed):
    """SDPA of one query over kk, vv [T, D] restricted to ``allowed`` [T] (bool)."""
    if not allowed.any():
        return np.zeros(qv.shape[-1])
    t = torch.from_numpy
    return F.scaled_dot_product_attention(t(qv)[None, None], t(kk)[None], t(vv)[None],
                                          attn_mask=t(allowed)[None, None])[0, 0].numpy()


def _token_allowed(len_b, block_sel, nblocks):
    """Token mask of a sequence from a per-block boolean vector (blocks past the
    sequence end select nothing)."""
    per_block = np.zeros(nblocks, bool)
    per_block[:len(block_sel)] = block_sel[:nblocks]
    return np.repeat(per_block, BLOCK)[:len_b]


# ---------------------------------------------------------------- mask form

def _mask_case(seed, lens, Hq, Hkv, D, nblocks, density):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    q, k, v = _rand((len(lens), Hq, D), seed + 1), _rand((T, Hkv, D), seed + 2), _rand((T, Hkv, D), seed + 3)
    bm = (rng.random((len(lens), Hkv, nblocks)) < density).astype(np.uint8)
    return cu, q, k, v, bm


@pytest.mark.parametrize("density", [1.0, 0.4])
def test_mask_form_matches_sdpa(density):
    lens = [130, 64, 257, 1]
    Hq, Hkv, D = 6, 2, 16
    nblocks = 6                       # more columns than the longest sequence has blocks
    cu, q, k, v, bm = _mask_case(11, lens, Hq, Hkv, D, nblocks, density)
    got = oa.decode_gqa_mask(q, k, v, cu, bm)
    G = Hq // Hkv
    for b, l in enumerate(lens):
        nbb = -(-l // BLOCK)
        for hq in range(Hq):
            kvh = hq // G
            allowed = _token_allowed(l, bm[b, kvh, :nbb] != 0, nbb)
            ref = _sdpa_one(q[b, hq], k[cu[b]:cu[b + 1], kvh], v[cu[b]:cu[b + 1], kvh], allowed)
            np.testing.assert_allclose(got[b, hq], ref, rtol=1e-12, atol=1e-12)


def test_mask_form_closed_forms():
    lens = [200, 70]
    Hq, Hkv, D = 4, 2, 8
    cu, q, k, _, bm = _mask_case(21, lens, Hq, Hkv, D, 5, 0.5)
    bm[0, 0] = 0                      # a (batch, KV head) with nothing selected
    bm[1, 1, :] = 0
    bm[1, 1, 4] = 1                   # only a block past the end: nothing selected either
    ones = np.ones((int(cu[-1]), Hkv, D))
    got = oa.decode_gqa_mask(q, k, ones, cu, bm)
    G = Hq // Hkv
    for b, l in enumerate(lens):
        nbb = -(-l // BLOCK)
        for hq in range(Hq):
            any_sel = (bm[b, hq // G, :nbb] != 0).any()
            np.testing.assert_allclose(got[b, hq], 1.0 if any_sel else 0.0, atol=1e-12)


def test_mask_form_single_block_is_that_block_alone():
    # one selected block: attention over exactly its tokens (ragged last block included)
    lens = [150]
    Hq, Hkv, D = 2, 1, 8
    cu, q, k, v, _ = _mask_case(31, lens, Hq, Hkv, D, 3, 0.0)
    for j in range(3):
        bm = np.zeros((1, 1, 3), np.uint8)
        bm[0, 0, j] = 1
        got = oa.decode_gqa_mask(q, k, v, cu, bm)
        lo, hi = BLOCK * j, min(BLOCK * j + BLOCK, lens[0])
        for hq in range(Hq):
            s = k[lo:hi, 0] @ q[0, hq] / np.sqrt(D)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(got[0, hq], p @ v[lo:hi, 0] / p.sum(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- paged KV

def _paged_case(seed, lens, Hkv, D, page_size, extra_pages):
    """Contiguous per-sequence K/V plus the same data scattered into shuffled pages."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    per_seq = [-(-l // page_size) for l in lens]
    mbps = max(per_seq) + 1
    num_pages = sum(per_seq) + extra_pages
    perm = rng.permutation(num_pages)
    table = np.full((B, mbps), -1, np.int64)
    kc = rng.standard_normal((num_pages, page_size, Hkv, D))
    vc = rng.standard_normal((num_pages, page_size, Hkv, D))
    ks, vs = [], []
    p = 0
    for b, l in enumerate(lens):
        kb, vb = rng.standard_normal((l, Hkv, D)), rng.standard_normal((l, Hkv, D))
        ks.append(kb)
        vs.append(vb)
        for lp in range(per_seq[b]):
            page = perm[p]
            p += 1
            table[b, lp] = page
            rows = np.arange(lp * page_size, min((lp + 1) * page_size, l))
            kc[page, rows - lp * page_size] = kb[rows]
            vc[page, rows - lp * page_size] = vb[rows]
    return kc, vc, table, ks, vs


@pytest.mark.parametrize("page_size", [64, 128, 256])
def test_paged_matches_sdpa_on_contiguous_copy(page_size):
    lens = [300, 64, 513]
    Hq, Hkv, D = 4, 2, 16
    kc, vc, table, ks, vs = _paged_case(41 + page_size, lens, Hkv, D, page_size, 3)
    rng = np.random.default_rng(5)
    q = _rand((len(lens), Hq, D), 42)
    ms = 7
    idx = np.full((len(lens), Hkv, ms), -1, np.int64)
    for b, l in enumerate(lens):
        nbb = -(-l // BLOCK)
        for h in range(Hkv):
            n = min(nbb, 4)
            idx[b, h, :n] = rng.choice(nbb, n, replace=False)
            idx[b, h, n] = nbb + 2          # out of range: selects nothing
    got = oa.decode_gqa_paged(q, kc, vc, np.array(lens), table, idx)
    G = Hq // Hkv
    for b, l in enumerate(lens):
        nbb = -(-l // BLOCK)
        for hq in range(Hq):
            sel = np.zeros(nbb, bool)
            for i in idx[b, hq // G]:
                if 0 <= i < nbb:
                    sel[i] = True
            allowed = _token_allowed(l, sel, nbb)
            ref = _sdpa_one(q[b, hq], ks[b][:, hq // G], vs[b][:, hq // G], allowed)
            np.testing.assert_allclose(got[b, hq], ref, rtol=1e-12, atol=1e-12)


def test_paged_bad_table_entries_select_nothing():
    lens = [256]
    Hq, Hkv, D, page_size = 2, 1, 8, 128
    kc, vc, table, ks, vs = _paged_case(51, lens, Hkv, D, page_size, 0)
    num_pages = kc.shape[0]
    q = _rand((1, Hq, D), 52)
    idx = np.array([[[0, 1, 2, 3]]])          # blocks 0,1 on logical page 0; 2,3 on page 1
    good = oa.decode_gqa_paged(q, kc, vc, np.array(lens), table, idx)
    bad = table.copy()
    bad[0, 1] = num_pages                     # page 1 points outside the cache
    got = oa.decode_gqa_paged(q, kc, vc, np.array(lens), bad, idx)
    only01 = oa.decode_gqa_paged(q, kc, vc, np.array(lens), table, np.array([[[0, 1, -1, -1]]]))
    np.testing.assert_allclose(got, only01, rtol=0, atol=0)
    assert not np.allclose(got, good)
    bad[0, 0] = -1
    bad[0, 1] = -7
    none = oa.decode_gqa_paged(q, kc, vc, np.array(lens), bad, idx)
    assert (none == 0).all()
