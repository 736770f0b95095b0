"""Pins for the mask and compaction oracle (CPU only).

Each check compares the oracle with something other than itself: hand-worked
fixtures, a brute-force rank count, torch.topk on tie-free data, closed-form
special cases and invariants."""
import os

import numpy as np
import pytest
import torch

from oracle import mask as om

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_blocks(path):
    """Parse a fixture: header lines followed by integer/float matrix rows."""
    out, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        toks = line.split()
        try:
            row = [float(t) for t in toks]
            cur[1].append(row)
        except ValueError:
            cur = (toks, [])
            out.append(cur)
    return out


def test_worked_topk_and_threshold_fixture():
    blocks = _read_blocks(os.path.join(GOLD, "mask_worked_4x4.txt"))
    assert blocks[0][0] == ["scores"]
    scores = np.array(blocks[0][1], dtype=np.float32)
    assert np.signbit(scores[3, 0]) and not np.signbit(scores[3, 1])  # -0.0 and 0.0
    scores = scores[None, None]
    n = 0
    for head, rows in blocks[1:]:
        kind, val, _, dense, _, diag = head
        want = np.array(rows, dtype=np.uint8)[None, None]
        if kind == "topk":
            got = om.build_mask_topk(scores, int(val), bool(int(dense)), bool(int(diag)))
        else:
            got = om.build_mask_threshold(scores, float(val), bool(int(dense)), bool(int(diag)))
        np.testing.assert_array_equal(got, want, err_msg=" ".join(head))
        n += 1
    assert n == 7


def _brute_topk(scores, topk, dense, diag):
    """Per-element rank count: column j is picked iff fewer than topk columns beat it,
    where c beats j when x_c > x_j, or x_c == x_j and c < j."""
    B, H, nb, _ = scores.shape
    m = np.zeros(scores.shape, np.uint8)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                x = [float(v) for v in scores[b, h, i]]
                for j in range(nb):
                    if dense and i >= nb - 2:
                        pick = True
                    else:
                        beat = sum(1 for c in range(nb) if x[c] > x[j] or (x[c] == x[j] and c < j))
                        pick = beat < topk
                    if j > i:
                        pick = False
                    if diag and j == i:
                        pick = True
                    m[b, h, i, j] = pick
    return m


@pytest.mark.parametrize("dense", [0, 1])
@pytest.mark.parametrize("diag", [0, 1])
def test_topk_matches_brute_force_with_ties(dense, diag):
    rng = np.random.default_rng(11)
    # Few distinct values so many ties occur.
    scores = rng.integers(-3, 4, size=(2, 3, 9, 9)).astype(np.float32)
    for topk in (0, 1, 3, 9):
        got = om.build_mask_topk(scores, topk, bool(dense), bool(diag))
        want = _brute_topk(scores, topk, dense, diag)
        np.testing.assert_array_equal(got, want)


def test_topk_matches_torch_topk_on_tie_free_scores():
    rng = np.random.default_rng(5)
    nb, topk = 40, 7
    scores = rng.permutation(2 * 3 * nb * nb).reshape(2, 3, nb, nb).astype(np.float32)
    got = om.build_mask_topk(scores, topk, False, False)
    t = torch.from_numpy(scores)
    idx = torch.topk(t, topk, dim=-1).indices
    ref = torch.zeros(t.shape, dtype=torch.bool).scatter_(-1, idx, True).tril_()
    np.testing.assert_array_equal(got, ref.numpy().astype(np.uint8))


def test_topk_invariants():
    rng = np.random.default_rng(3)
    nb, topk = 33, 5
    scores = rng.standard_normal((2, 2, nb, nb), dtype=np.float32)
    raw = om.build_mask_topk(scores, topk, False, False)
    # The last row keeps every column after tril, so it has exactly topk picks.
    assert (raw[..., nb - 1, :].sum(-1) == topk).all()
    # Subset of the lower triangle; at most topk per row.
    assert (np.triu(raw, 1) == 0).all()
    assert (raw.sum(-1) <= topk).all()
    full = om.build_mask_topk(scores, topk, True, True)
    d = np.arange(nb)
    assert (full[..., d, d] == 1).all()
    tri = np.tril(np.ones((nb, nb), np.uint8))
    np.testing.assert_array_equal(full[..., nb - 2:, :], np.broadcast_to(tri[nb - 2:], full[..., nb - 2:, :].shape))
    # Forcing the diagonal / dense rows only adds blocks.
    assert ((full.astype(int) - raw.astype(int)) >= 0).all()


def test_special_cases():
    rng = np.random.default_rng(4)
    nb = 17
    scores = rng.standard_normal((1, 2, nb, nb), dtype=np.float32)
    tri = np.broadcast_to(np.tril(np.ones((nb, nb), np.uint8)), scores.shape)
    eye = np.broadcast_to(np.eye(nb, dtype=np.uint8), scores.shape)
    np.testing.assert_array_equal(om.build_mask_topk(scores, nb, False, False), tri)
    np.testing.assert_array_equal(om.build_mask_threshold(scores, -np.inf, False, False), tri)
    np.testing.assert_array_equal(om.build_mask_threshold(scores, np.inf, False, True), eye)
    np.testing.assert_array_equal(om.build_mask_topk(scores, 0, False, True), eye)
    # threshold keeps strictly greater only
    s2 = np.full((1, 1, 3, 3), 0.5, np.float32)
    assert om.build_mask_threshold(s2, 0.5, False, False).sum() == 0
    assert om.build_mask_threshold(s2, np.nextafter(np.float32(0.5), np.float32(0)), False, False).sum() == 6


def test_nb_one_and_two():
    s = np.array([[[[0.3]]]], np.float32)
    assert om.build_mask_topk(s, 0, False, False).sum() == 0
    assert om.build_mask_topk(s, 1, False, False).sum() == 1
    assert om.build_mask_topk(s, 0, True, False).sum() == 1  # dense last rows cover row 0
    s2 = np.zeros((1, 1, 2, 2), np.float32)
    np.testing.assert_array_equal(om.build_mask_threshold(s2, 1.0, True, False)[0, 0], [[1, 0], [1, 1]])


def test_compaction_fixture():
    blocks = _read_blocks(os.path.join(GOLD, "compaction_worked.txt"))
    mask = np.array(blocks[0][1], dtype=np.uint8)[None, None]
    for head, _ in blocks[1:]:
        pass
    # Fixture layout: "causal c" header, then lines "idx ... cnt n".
    lines = [l.split("#", 1)[0].strip() for l in open(os.path.join(GOLD, "compaction_worked.txt"))]
    lines = [l for l in lines if l]
    causal = None
    want = {0: [], 1: []}
    for l in lines:
        t = l.split()
        if t[0] == "causal":
            causal = int(t[1])
        elif t[0] == "idx":
            k = t.index("cnt")
            want[causal].append(([int(x) for x in t[1:k]], int(t[k + 1])))
    for c in (0, 1):
        idx, cnt = om.mask_to_indices(mask, bool(c))
        assert [list(r) for r in idx[0, 0]] == [w[0] for w in want[c]]
        assert list(cnt[0, 0]) == [w[1] for w in want[c]]


def test_compaction_round_trip():
    rng = np.random.default_rng(8)
    mask = (rng.random((2, 3, 21, 21)) < 0.3).astype(np.uint8) * rng.integers(1, 255, (2, 3, 21, 21)).astype(np.uint8)
    for causal in (False, True):
        idx, cnt = om.mask_to_indices(mask, causal)
        nb = mask.shape[-1]
        sel = mask != 0
        if causal:
            sel &= np.tril(np.ones((nb, nb), bool))
        np.testing.assert_array_equal(cnt, sel.sum(-1))
        back = np.zeros(mask.shape, bool)
        for b in range(2):
            for h in range(3):
                for i in range(nb):
                    row = idx[b, h, i]
                    c = cnt[b, h, i]
                    assert (row[c:] == -1).all()
                    assert (np.diff(row[:c]) > 0).all()
                    back[b, h, i, row[:c]] = True
        np.testing.assert_array_equal(back, sel)
