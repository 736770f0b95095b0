"""Pins for the attention oracle (CPU only).

The oracle is checked against torch's scaled_dot_product_attention in float64
(a library routine), scalar brute force on tiny shapes, closed forms and
hand-worked fixtures."""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as oa

GOLD = os.path.join(os.path.dirname(__file__), "golden")
BLOCK = 64


def _kron_mask(block_mask, S, causal):
    tok = np.kron(block_mask, np.ones((BLOCK, BLOCK)))[..., :S, :S] != 0
    if causal:
        tok &= np.tril(np.ones((S, S), bool))
    return tok


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_true_mask_is_dense_causal_sdpa():
    B, H, S, D = 1, 2, 200, 32
    q, k, v = (_rand((B, H, S, D), s) for s in (1, 2, 3))
    nb = -(-S // BLOCK)
    mask = np.ones((B, H, nb, nb), np.uint8)
    got = oa.prefill(q, k, v, mask, True)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)), is_causal=True).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    got_nc = oa.prefill(q, k, v, mask, False)
    ref_nc = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v))).numpy()
    np.testing.assert_allclose(got_nc, ref_nc, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_random_mask_matches_sdpa_with_expanded_mask(causal):
    B, H, S, D = 2, 2, 300, 16
    q, k, v = (_rand((B, H, S, D), s) for s in (4, 5, 6))
    nb = -(-S // BLOCK)
    rng = np.random.default_rng(7)
    mask = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    mask[..., np.arange(nb), np.arange(nb)] = 1   # keep every row non-empty for SDPA
    got = oa.prefill(q, k, v, mask, causal)
    tok = _kron_mask(mask, S, causal)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                         attn_mask=torch.from_numpy(tok)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def _brute_prefill(q, k, v, mask, causal):
    S, D = q.shape
    out = np.zeros((S, D))
    for r in range(S):
        ws, acc = [], None
        keys = [t for t in range(S) if mask[r // BLOCK][t // BLOCK] and (not causal or t <= r)]
        if not keys:
            continue
        ss = [sum(q[r, d] * k[t, d] for d in range(D)) / math.sqrt(D) for t in keys]
        mx = max(ss)
        ws = [math.exp(s - mx) for s in ss]
        tot = sum(ws)
        for d in range(D):
            out[r, d] = sum(w * v[t, d] for w, t in zip(ws, keys)) / tot
    return out


def test_all_lower_triangular_masks_nb3_brute_force():
    S, D = 150, 3   # nb = 3 with a ragged last block
    q, k, v = (_rand((S, D), s) for s in (9, 10, 11))
    lower = [(i, j) for i in range(3) for j in range(i + 1)]
    for bits in itertools.product([0, 1], repeat=len(lower)):
        m = np.zeros((3, 3), np.uint8)
        for (i, j), b in zip(lower, bits):
            m[i, j] = b
        got = oa.prefill_head_rows(q, k, v, m, True)
        want = _brute_prefill(q, k, v, m, True)
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12, err_msg=str(bits))


def test_noncausal_upper_blocks_brute_force():
    S, D = 130, 2
    q, k, v = (_rand((S, D), s) for s in (12, 13, 14))
    m = np.array([[0, 1, 1], [1, 0, 0], [0, 0, 1]], np.uint8)
    np.testing.assert_allclose(oa.prefill_head_rows(q, k, v, m, False), _brute_prefill(q, k, v, m, False),
                               rtol=1e-10, atol=1e-12)


def test_closed_forms():
    S, D = 256, 8
    q, k = _rand((S, D), 20), _rand((S, D), 21)
    nb = S // BLOCK
    rng = np.random.default_rng(22)
    m = (rng.random((nb, nb)) < 0.4).astype(np.uint8)
    m[1, :] = 0                    # an empty row block
    m[0, 0] = 1
    ones = np.ones((S, D))
    out = oa.prefill_head_rows(q, k, ones, m, True)
    nonempty = np.array([(m[r // BLOCK, : r // BLOCK + 1] != 0).any() for r in range(S)])
    # softmax rows sum to one: V = 1 gives 1 on non-empty rows, 0 on empty rows
    np.testing.assert_allclose(out[nonempty], 1.0, rtol=0, atol=1e-13)
    assert (out[~nonempty] == 0).all()
    # one-hot V recovers the probabilities, which are >= 0 and sum to one
    eye = np.eye(S)
    P = oa.prefill_head_rows(q, k, eye, m, True)
    assert (P >= 0).all()
    np.testing.assert_allclose(P[nonempty].sum(-1), 1.0, atol=1e-13)
    assert (np.triu(P, 1) == 0).all()        # causal: nothing above the diagonal
    # row 0 sees only key 0
    v = _rand((S, D), 23)
    np.testing.assert_allclose(oa.prefill_head_rows(q, k, v, m, True)[0], v[0], atol=1e-14)
    # q = 0: the mean of the allowed values
    z = oa.prefill_head_rows(np.zeros((S, D)), k, v, m, True)
    for r in (5, 70, 200, 255):
        keys = [t for t in range(r + 1) if m[r // BLOCK, t // BLOCK]]
        if keys:
            np.testing.assert_allclose(z[r], v[keys].mean(0), atol=1e-13)


def test_diagonal_only_is_blockwise_causal_sdpa():
    S, D = 192, 16
    q, k, v = (_rand((S, D), s) for s in (30, 31, 32))
    m = np.eye(S // BLOCK, dtype=np.uint8)
    got = oa.prefill_head_rows(q, k, v, m, True)
    for c in range(S // BLOCK):
        sl = slice(c * BLOCK, (c + 1) * BLOCK)
        ref = F.scaled_dot_product_attention(*(torch.from_numpy(x[sl])[None] for x in (q, k, v)),
                                             is_causal=True)[0].numpy()
        np.testing.assert_allclose(got[sl], ref, rtol=1e-12, atol=1e-12)


def _fixture_lines():
    out = []
    for l in open(os.path.join(GOLD, "attention_worked.txt")):
        l = l.split("#", 1)[0].strip()
        if l:
            out.append(l.split())
    return out


def _vals(toks):
    return [float(t) for t in toks]


def test_worked_prefill_fixture():
    L = _fixture_lines()
    get = {tuple(t[:2]): t[2:] for t in L if t[0] == "prefill" and t[1] in ("q", "k_weights", "v")}
    q = np.array(_vals(get[("prefill", "q")]))[:, None]
    k = np.log(np.array(_vals(get[("prefill", "k_weights")])))[:, None]
    v = np.array(_vals(get[("prefill", "v")]))[:, None]
    n = 0
    for t in L:
        if t[0] == "prefill" and t[1] == "causal":
            causal, mval = int(t[2]), int(t[4])
            want = np.array(_vals(t[6:]))
            got = oa.prefill_head_rows(q, k, v, np.array([[mval]], np.uint8), bool(causal))[:, 0]
            np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
            n += 1
    assert n == 3


def test_worked_decode_and_merge_fixture():
    L = _fixture_lines()
    get = {tuple(t[:2]): t[2:] for t in L if t[0] == "decode" and t[1] in ("q", "k_weights", "v")}
    q = np.array(_vals(get[("decode", "q")]))[None, :, None]                 # [1, 2, 1]
    k = np.log(np.array(_vals(get[("decode", "k_weights")])))[:, None, None]  # [3, 1, 1]
    v = np.array(_vals(get[("decode", "v")]))[:, None, None]
    cu = np.array([0, 3])
    n = 0
    for t in L:
        if t[0] == "decode" and t[1] == "indices":
            e = t.index("expect")
            idx = np.array([int(x) for x in t[2:e]])[None, None, :]
            got = oa.decode_gqa(q, k, v, cu, idx)[0, :, 0]
            np.testing.assert_allclose(got, _vals(t[e + 1:]), rtol=1e-14, atol=1e-14)
            n += 1
        elif t[0] == "gqa":
            T, D = 70, 4
            kk = _rand((T, 2, D), 40)
            vv = np.empty((T, 2, D))
            vv[:, 0], vv[:, 1] = 5.0, -3.0
            qq = _rand((1, 4, D), 41)
            got = oa.decode_gqa(qq, kk, vv, np.array([0, T]), np.array([[[1, 0]], [[0, -1]]]).reshape(1, 2, 2))
            np.testing.assert_allclose(got[0, :, 0], _vals(t[2:]), atol=1e-14)
            n += 1
        elif t[0] == "merge":
            i_lse, i_exp = t.index("lse"), t.index("expect")
            o = np.array(_vals(t[2:i_lse]))[:, None]
            lse = np.array(_vals(t[i_lse + 1:i_exp]))
            got = oa.merge_partials(o, lse)
            np.testing.assert_allclose(got, _vals(t[i_exp + 1:]), rtol=1e-14)
            n += 1
    assert n == 5


def test_decode_all_blocks_is_dense_single_query_sdpa():
    B, Hq, Hkv, D = 3, 8, 2, 32
    lens = [130, 64, 257]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q, k, v = _rand((B, Hq, D), 50), _rand((T, Hkv, D), 51), _rand((T, Hkv, D), 52)
    nbmax = max(-(-l // BLOCK) for l in lens)
    idx = np.full((B, Hkv, nbmax + 2), -1, np.int32)
    for b, l in enumerate(lens):
        nbb = -(-l // BLOCK)
        idx[b, :, :nbb] = np.arange(nbb)[::-1]
    idx[0, 1, -1] = 999   # out-of-range index selects nothing
    got = oa.decode_gqa(q, k, v, cu, idx)
    G = Hq // Hkv
    for b, l in enumerate(lens):
        kk = torch.from_numpy(k[cu[b]:cu[b + 1]]).permute(1, 0, 2).repeat_interleave(G, 0)
        vv = torch.from_numpy(v[cu[b]:cu[b + 1]]).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b])[:, None], kk, vv)[:, 0].numpy()
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-12)


def test_decode_equals_prefill_last_row():
    # Same keys, block list = the last query block's mask row, len a multiple of 64.
    S, D, Hkv, G = 256, 16, 2, 3
    nb = S // BLOCK
    k, v = _rand((S, Hkv, D), 60), _rand((S, Hkv, D), 61)
    q = _rand((1, Hkv * G, D), 62)
    rng = np.random.default_rng(63)
    sel = [sorted(rng.choice(nb - 1, 2, replace=False).tolist() + [nb - 1], reverse=True) for _ in range(Hkv)]
    idx = np.array(sel, np.int32)[None]
    got = oa.decode_gqa(q, k, v, np.array([0, S]), idx)
    for hq in range(Hkv * G):
        kvh = hq // G
        m = np.zeros((nb, nb), np.uint8)
        m[nb - 1, sel[kvh]] = 1
        qq = np.zeros((S, D))
        qq[S - 1] = q[0, hq]
        row = oa.prefill_head_rows(qq, k[:, kvh], v[:, kvh], m, True, rows=[S - 1])[0]
        np.testing.assert_allclose(got[0, hq], row, rtol=1e-12, atol=1e-12)


def test_decode_split_merge_reproduces_unsplit():
    # Split the selected tokens into parts, compute each part's normalised
    # output and base-2 log-sum-exp, and merge: must equal the unsplit result.
    D, T = 8, 300
    q = _rand((D,), 70)
    k, v = _rand((T, D), 71), _rand((T, D), 72)
    s = k @ q / math.sqrt(D)
    full = np.exp(s - s.max()) @ v / np.exp(s - s.max()).sum()
    parts = [np.arange(0, 70), np.arange(70, 71), np.arange(71, 300), np.arange(0)]
    o_parts, lse = [], []
    for p in parts:
        if p.size == 0:
            o_parts.append(np.zeros(D))
            lse.append(-np.inf)
            continue
        sp = s[p]
        m = sp.max()
        w = np.exp(sp - m)
        o_parts.append(w @ v[p] / w.sum())
        lse.append((m + math.log(w.sum())) / math.log(2.0))
    got = oa.merge_partials(np.array(o_parts), np.array(lse))
    np.testing.assert_allclose(got, full, rtol=1e-12, atol=1e-13)
    assert (oa.merge_partials(np.zeros((3, D)), np.full(3, -np.inf)) == 0).all()


def test_decode_length_mask_and_padding():
    # The last block of a ragged sequence stops at len_b; -1 and out-of-range
    # indices are skipped; order is irrelevant.
    D = 4
    lens = [100]
    T = 100
    q, k, v = _rand((1, 1, D), 80), _rand((T, 1, D), 81), _rand((T, 1, D), 82)
    cu = np.array([0, T])
    a = oa.decode_gqa(q, k, v, cu, np.array([[[1, -1, 0, 7]]]))
    b = oa.decode_gqa(q, k, v, cu, np.array([[[0, 1, -1, -1]]]))
    np.testing.assert_allclose(a, b, rtol=1e-15)
    assert oa.decode_allowed_tokens(100, [1]).tolist() == list(range(64, 100))
    assert oa.decode_allowed_tokens(100, [2, -1]).tolist() == []
