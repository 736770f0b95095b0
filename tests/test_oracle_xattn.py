"""Pins for the XAttention estimator oracle (CPU only).

Checked against the guide's worked selection example and hand-worked rows
(tests/golden), brute-force loops, torch's softmax on the token grid (stride
1), closed forms (row totals, constant keys) and invariants of the rule."""
import itertools
import os

import numpy as np
import pytest
import torch

from oracle import xattn as ox

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    out, cur = [], None
    for line in open(os.path.join(GOLD, "xattn_selection_example.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        toks = line.split()
        if toks[0] == "case":
            cur = [float(toks[1])] + [int(t) for t in toks[2:5]]
            out.append([cur, None, None])
        elif out[-1][1] is None:
            out[-1][1] = np.array([float(t) for t in toks], np.float32)
        else:
            out[-1][2] = np.array([int(t) for t in toks], np.uint8)
    return out


def test_worked_selection_fixture():
    cases = _cases()
    assert len(cases) == 8
    for (thr, sink, diag, last), w, want in cases:
        got = ox.find_blocks_row(w, thr, None if sink < 0 else sink, None if diag < 0 else diag,
                                 None if last < 0 else last)
        np.testing.assert_array_equal(got, want, err_msg=f"thr={thr} sink={sink} diag={diag}")


def _rng(seed):
    return np.random.default_rng(seed)


def test_stride_reshape_layout():
    # stride 8 as the guide lists it: K' row t' starts with key row 8t' and
    # ends with 8t'+7; Q' row r' starts with query row 8r'+7 and ends with 8r'.
    q = _rng(1).standard_normal((2, 64, 3))
    k = _rng(2).standard_normal((2, 40, 3))
    qr, kr = ox.stride_reshape(q, k, 8)
    assert qr.shape == (2, 8, 24) and kr.shape == (2, 5, 24)
    for t in range(5):
        for j in range(8):
            np.testing.assert_array_equal(kr[:, t, 3 * j:3 * j + 3], k[:, 8 * t + j])
    for r in range(8):
        for j in range(8):
            np.testing.assert_array_equal(qr[:, r, 3 * j:3 * j + 3], q[:, 8 * r + 7 - j])
    # K' is the contiguous reshape of K; Q' the same with each group reversed
    np.testing.assert_array_equal(kr, k.reshape(2, 5, 24))
    np.testing.assert_array_equal(qr, q.reshape(2, 8, 8, 3)[:, :, ::-1, :].reshape(2, 8, 24))


def _brute_block_sums(q, k, s, norm, causal):
    """Scalar loops: pair sums, softmax and block sums written out."""
    Sq, D = q.shape
    Sk = k.shape[0]
    rq, rk = Sq // s, Sk // s
    past = (Sk - Sq) // s
    b = 64 // s
    nbq, nbk = -(-Sq // 64), -(-Sk // 64)
    out = np.zeros((nbq, nbk))
    for r in range(rq):
        logit = []
        for t in range(rk):
            if causal and t > r + past:
                logit.append(None)
                continue
            acc = 0.0
            for j in range(s):
                qa = q[r * s + s - 1 - j]
                ka = k[t * s + j]
                for d in range(D):
                    acc += qa[d] * ka[d]
            logit.append(acc / (np.sqrt(D) * s * norm))
        mx = max(x for x in logit if x is not None)
        e = [0.0 if x is None else np.exp(x - mx) for x in logit]
        tot = sum(e)
        for t in range(rk):
            out[r // b, t // b] += e[t] / tot
    return out


@pytest.mark.parametrize("s,Sq,Sk,causal,norm", [(4, 128, 128, True, 1.0), (8, 192, 192, False, 1.0),
                                                  (16, 64, 192, True, 0.7), (4, 72, 200, True, 1.5),
                                                  (8, 200, 200, True, 1.0)])
def test_block_sums_brute_force(s, Sq, Sk, causal, norm):
    D = 3
    q = _rng(s + Sq).standard_normal((Sq, D))
    k = _rng(s + Sk + 1).standard_normal((Sk, D))
    got = ox.block_sums(q[None], k[None], s, norm, causal)[0]
    np.testing.assert_allclose(got, _brute_block_sums(q, k, s, norm, causal), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_stride_one_is_token_softmax_block_mass(causal):
    # stride 1: the logits are plain scaled dot products; block sums are the
    # 64x64 block sums of torch's softmax attention weights
    B, H, S, D = 1, 2, 200, 8
    q = _rng(3).standard_normal((B, H, S, D))
    k = _rng(4).standard_normal((B, H, S, D))
    got = ox.block_sums(q, k, 1, 1.0, causal)
    lg = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) / np.sqrt(D)
    if causal:
        lg = lg.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    p = torch.softmax(lg, dim=-1).numpy()
    nb = -(-S // 64)
    want = np.zeros((B, H, nb, nb))
    for i in range(nb):
        for j in range(nb):
            want[..., i, j] = p[..., 64 * i:64 * i + 64, 64 * j:64 * j + 64].sum(axis=(-1, -2))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("s", [4, 8, 16])
def test_row_totals_and_constant_keys(s):
    Sq = Sk = 448 + s * 3          # ragged last block
    D = 4
    q = _rng(5).standard_normal((1, 1, Sq, D))
    k = _rng(6).standard_normal((1, 1, Sk, D))
    got = ox.block_sums(q, k, s)[0, 0]
    rows = Sq // s
    b = 64 // s
    want_tot = [min(b, rows - qi * b) for qi in range(got.shape[0])]
    np.testing.assert_allclose(got.sum(axis=-1), want_tot, rtol=1e-12)
    # identical key rows: every visible reshaped key gets the same weight
    kc = np.repeat(k[:, :, :1, :], Sk, axis=2)
    got = ox.block_sums(q, kc, s)[0, 0]
    want = np.zeros_like(got)
    for r in range(rows):
        vis = r + 1
        for t in range(vis):
            want[r // b, t // b] += 1.0 / vis
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)


def test_norm_divides_the_logits():
    q = _rng(7).standard_normal((1, 1, 256, 8))
    k = _rng(8).standard_normal((1, 1, 256, 8))
    np.testing.assert_allclose(ox.block_sums(q, k, 8, norm=2.0), ox.block_sums(q / 2, k, 8, norm=1.0),
                               rtol=1e-12, atol=1e-15)
    # a large norm flattens the estimate toward the constant-key closed form
    flat = ox.block_sums(q, k, 8, norm=1e9)
    kc = np.repeat(k[:, :, :1, :], 256, axis=2)
    np.testing.assert_allclose(flat, ox.block_sums(q, kc, 8), atol=1e-7)


def test_chunk_rows_are_the_last_rows_of_the_square_estimate():
    S, Sq, D = 320, 128, 4
    q = _rng(9).standard_normal((1, 2, S, D))
    k = _rng(10).standard_normal((1, 2, S, D))
    full = ox.block_sums(q, k, 8)
    chunk = ox.block_sums(q[:, :, S - Sq:], k, 8)
    np.testing.assert_allclose(chunk, full[:, :, -(Sq // 64):], rtol=1e-12, atol=1e-15)


def _prefix_rule(w, thr, forced, last):
    """Independent statement: the smallest weight-ranked prefix of the
    unforced columns whose sum reaches thr * total (all of them if none does),
    plus the forced columns, cut after `last`."""
    w = w.astype(np.float64)
    n = len(w)
    total = float(np.sum(w))
    free = [c for c in range(n) if c not in forced]
    ranked = sorted(free, key=lambda c: (-w[c], c)) + sorted(forced)
    keep = set(forced)
    acc = 0.0
    for c in ranked:
        if acc >= thr * total:
            break
        keep.add(c)
        acc += w[c] if c not in forced else 0.0
    m = np.zeros(n, np.uint8)
    m[list(keep)] = 1
    if last is not None:
        m[last + 1:] = 0
    return m


def test_selection_matches_prefix_rule_on_random_rows():
    rng = _rng(11)
    for trial in range(400):
        n = int(rng.integers(1, 40))
        # weights on a 1/1024 grid: every sum is exact, so the rule is exact
        w = (rng.integers(0, 64, n) / 1024.0).astype(np.float32)
        thr = float(rng.choice([0.0, 0.3, 0.5, 0.9, 0.95, 1.0]))
        sink = 0 if rng.random() < 0.5 else None
        diag = int(rng.integers(0, n)) if rng.random() < 0.7 else None
        last = diag if (diag is not None and rng.random() < 0.5) else None
        forced = {c for c in (sink, diag) if c is not None}
        got = ox.find_blocks_row(w, thr, sink, diag, last)
        np.testing.assert_array_equal(got, _prefix_rule(w, thr, forced, last), err_msg=f"trial {trial}")


def test_selection_invariants():
    rng = _rng(12)
    sums = rng.random((2, 3, 6, 9)).astype(np.float32)
    past = 3
    for i in range(6):
        sums[..., i, i + past + 1:] = 0   # an estimate gives no weight after the diagonal
    m = ox.find_blocks(sums, 0.8, True, True, True)
    for i in range(6):
        assert (m[..., i, 0] == 1).all() and (m[..., i, i + past] == 1).all()
        assert (m[..., i, i + past + 1:] == 0).all()
    # kept unforced weight reaches the threshold, and is a top-ranked set
    for b, h, i in itertools.product(range(2), range(3), range(6)):
        d = i + past
        w = sums[b, h, i].astype(np.float64)
        kept = [c for c in range(9) if m[b, h, i, c] and c not in (0, d)]
        dropped = [c for c in range(d + 1) if not m[b, h, i, c]]
        if dropped:
            assert min(w[kept]) >= max(w[dropped])
            assert w[kept].sum() >= 0.8 * w.sum() - 1e-12
    # threshold 0: only the forced columns; threshold 1: every column up to the diagonal
    m0 = ox.find_blocks(sums, 0.0, True, True, True)
    m1 = ox.find_blocks(sums, 1.0, False, False, True)
    for i in range(6):
        want0 = np.zeros(9, np.uint8)
        want0[[0, i + past]] = 1
        assert (m0[..., i, :] == want0).all()
        assert (m1[..., i, :i + past + 1] == 1).all() and (m1[..., i, i + past + 1:] == 0).all()


def test_estimate_mask_keeps_most_of_the_mass():
    q = _rng(13).standard_normal((1, 2, 512, 16))
    k = _rng(14).standard_normal((1, 2, 512, 16))
    bs, m = ox.estimate_mask(q, k, 8, 1.0, 0.9, True, True, True)
    kept = (bs * m).sum(axis=-1)
    assert (kept >= 0.9 * bs.sum(axis=-1) - 1e-6).all()
    assert (np.triu(m, 1) == 0).all()
