"""Pins for the decode oracles with a value head dim different from the key
head dim (the guide's decode takes dim and dim_v, §9.2) and with query-head
groups up to 64 (§6.1: up to 64 query heads per KV head share one m-block).

Checked against torch's scaled_dot_product_attention in float64 (a library
routine that accepts a value width different from the key width) on token
masks the tests build themselves, and against closed forms."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as oa

BLOCK = 64


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(qv, kk, vv):
    t = torch.from_numpy
    return F.scaled_dot_product_attention(t(qv)[None, None], t(kk)[None], t(vv)[None])[0, 0].numpy()


def _tokens(len_b, blocks):
    sel = np.zeros(-(-len_b // BLOCK), bool)
    for i in blocks:
        if 0 <= i < sel.size:
            sel[i] = True
    return np.nonzero(np.repeat(sel, BLOCK)[:len_b])[0]


@pytest.mark.parametrize("D,Dv,Hq,Hkv", [(64, 128, 8, 2), (128, 64, 64, 1), (32, 48, 64, 2),
                                         (16, 8, 96, 3)])
def test_index_form_matches_sdpa(D, Dv, Hq, Hkv):
    lens = [130, 64, 257, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand((len(lens), Hq, D), 1), _rand((T, Hkv, D), 2), _rand((T, Hkv, Dv), 3)
    rng = np.random.default_rng(4)
    idx = np.full((len(lens), Hkv, 6), -1, np.int32)
    for b, l in enumerate(lens):
        nbb = -(-l // BLOCK)
        for h in range(Hkv):
            n = int(rng.integers(1, nbb + 1))
            idx[b, h, :n] = rng.choice(nbb, size=n, replace=False)
    got = oa.decode_gqa(q, k, v, cu, idx)
    assert got.shape == (len(lens), Hq, Dv)
    G = Hq // Hkv
    for b, l in enumerate(lens):
        for hq in range(Hq):
            toks = cu[b] + _tokens(l, idx[b, hq // G])
            want = _sdpa(q[b, hq], k[toks, hq // G], v[toks, hq // G])
            np.testing.assert_allclose(got[b, hq], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Dv", [8, 128])
def test_mask_form_matches_sdpa(Dv):
    lens = [200, 64, 3]
    Hq, Hkv, D = 64, 2, 16
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand((len(lens), Hq, D), 5), _rand((T, Hkv, D), 6), _rand((T, Hkv, Dv), 7)
    bm = (np.random.default_rng(8).random((len(lens), Hkv, 5)) < 0.6).astype(np.uint8)
    bm[:, :, 0] = 1
    got = oa.decode_gqa_mask(q, k, v, cu, bm)
    G = Hq // Hkv
    for b, l in enumerate(lens):
        for hq in range(Hq):
            toks = cu[b] + _tokens(l, np.nonzero(bm[b, hq // G])[0])
            np.testing.assert_allclose(got[b, hq], _sdpa(q[b, hq], k[toks, hq // G], v[toks, hq // G]),
                                       rtol=1e-12, atol=1e-12)


def test_paged_form_matches_sdpa():
    rng = np.random.default_rng(9)
    lens = np.array([300, 129])
    Hq, Hkv, D, Dv, page = 32, 1, 16, 24, 128
    per = [-(-int(l) // page) for l in lens]
    num_pages = sum(per) + 2
    perm = rng.permutation(num_pages)
    kc, vc = _rand((num_pages, page, Hkv, D), 10), _rand((num_pages, page, Hkv, Dv), 11)
    table = np.full((2, max(per)), -1, np.int32)
    p = 0
    for b in range(2):
        for lp in range(per[b]):
            table[b, lp] = perm[p]
            p += 1
    idx = np.array([[[4, 0, 2, -1]], [[2, 1, -1, -1]]], np.int32)
    q = _rand((2, Hq, D), 12)
    got = oa.decode_gqa_paged(q, kc, vc, lens.astype(np.int32), table, idx)
    assert got.shape == (2, Hq, Dv)
    for b in range(2):
        toks = _tokens(int(lens[b]), idx[b, 0])
        pages, rows = table[b, toks // page], toks % page
        for hq in range(Hq):
            np.testing.assert_allclose(got[b, hq], _sdpa(q[b, hq], kc[pages, rows, 0], vc[pages, rows, 0]),
                                       rtol=1e-12, atol=1e-12)


def test_closed_forms_with_wide_values():
    cu = np.array([0, 150])
    Hq, Hkv, D, Dv = 64, 1, 8, 40
    q, k = _rand((1, Hq, D), 13), _rand((150, Hkv, D), 14)
    idx = np.array([[[2, 0, -1]]], np.int32)
    # V = 1 everywhere: softmax weights sum to 1, so every output is 1
    got = oa.decode_gqa(q, k, np.ones((150, Hkv, Dv)), cu, idx)
    np.testing.assert_allclose(got, 1.0, rtol=1e-14)
    # V carries the token position: the output is the softmax-weighted mean position,
    # which lies inside the selected tokens' range
    pos = np.repeat(np.arange(150.0)[:, None, None], Dv, axis=2)
    got = oa.decode_gqa(q, k, pos, cu, idx)
    assert ((got >= 0) & (got <= 149)).all()
    # q = 0: uniform weights over the selected tokens (0..63 and 128..149)
    toks = np.r_[0:64, 128:150]
    got = oa.decode_gqa(np.zeros((1, Hq, D)), k, pos, cu, idx)
    np.testing.assert_allclose(got, toks.mean(), rtol=1e-14)
