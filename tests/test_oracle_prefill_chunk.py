"""Pins for the prefill oracle with fewer queries than keys (Sq < Sk, CPU only).

The queries are the last Sq positions of an Sk-token context.  Checked
against torch's scaled_dot_product_attention in float64 with a token mask the
test builds itself, against the last rows of the square problem, and against
closed forms."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as oa

BLOCK = 64


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _token_mask(block_mask, Sq, Sk, causal):
    tok = np.repeat(np.repeat(block_mask != 0, BLOCK, axis=-2), BLOCK, axis=-1)[..., :Sq, :Sk]
    if causal:
        past = Sk - Sq
        tok = tok & (np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + past)
    return tok


@pytest.mark.parametrize("Sq,Sk", [(64, 256), (100, 300), (37, 37), (130, 451), (1, 200)])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_matches_sdpa_with_token_mask(Sq, Sk, causal):
    B, H, D = 1, 2, 16
    q, k, v = _rand((B, H, Sq, D), 1), _rand((B, H, Sk, D), 2), _rand((B, H, Sk, D), 3)
    nbq, nbk = -(-Sq // BLOCK), -(-Sk // BLOCK)
    rng = np.random.default_rng(Sq * 7 + Sk)
    m = (rng.random((B, H, nbq, nbk)) < 0.5).astype(np.uint8)
    m[..., :, 0] = 1                  # every query row keeps key 0, so SDPA sees no empty row
    got = oa.prefill(q, k, v, m, causal)
    tok = _token_mask(m, Sq, Sk, causal)
    assert tok.any(axis=-1).all()
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                         attn_mask=torch.from_numpy(tok)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_chunk_equals_last_rows_of_the_square_problem():
    # past a multiple of 64: the chunk's block rows are the square mask's last rows
    Sk, Sq, D = 320, 128, 8
    q_full, k, v = _rand((Sk, D), 10), _rand((Sk, D), 11), _rand((Sk, D), 12)
    nbk = Sk // BLOCK
    rng = np.random.default_rng(13)
    m_full = np.tril((rng.random((nbk, nbk)) < 0.6).astype(np.uint8))
    m_full[np.arange(nbk), np.arange(nbk)] = 1
    full = oa.prefill_head_rows(q_full, k, v, m_full, True)
    chunk = oa.prefill_head_rows(q_full[Sk - Sq:], k, v, m_full[nbk - Sq // BLOCK:], True)
    np.testing.assert_allclose(chunk, full[Sk - Sq:], rtol=1e-12, atol=1e-14)


def test_chunk_closed_forms():
    Sq, Sk, D = 90, 250, 8
    q, k = _rand((Sq, D), 20), _rand((Sk, D), 21)
    nbq, nbk = 2, 4
    m = np.zeros((nbq, nbk), np.uint8)
    m[0, 3] = 1                        # causally invisible for every row of block 0 except its tail
    m[1, 1] = 1
    got = oa.prefill_head_rows(q, k, np.ones((Sk, D)), m, True)
    past = Sk - Sq
    for r in range(Sq):
        keys = [t for t in range(Sk) if m[r // BLOCK, t // BLOCK] and t <= r + past]
        np.testing.assert_allclose(got[r], 1.0 if keys else 0.0, atol=1e-12)
    # one visible key: the output is that key's value row
    v = _rand((Sk, D), 22)
    m1 = np.zeros((1, nbk), np.uint8)
    m1[0, 3] = 1
    q1 = _rand((1, D), 23)
    got1 = oa.prefill_head_rows(q1, k, v, m1, True)      # row 0 sits at position Sk - 1
    s = k[192:250] @ q1[0] / np.sqrt(D)
    p = np.exp(s - s.max())
    np.testing.assert_allclose(got1[0], p @ v[192:250] / p.sum(), rtol=1e-12, atol=1e-12)
