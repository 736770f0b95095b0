"""GPU parity: prefill with fewer queries than keys (Sq <= Sk) against the float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _case(B, H, Sq, Sk, D, seed, density=0.4):
    rng = np.random.default_rng(seed)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sq, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    nbq, nbk = -(-Sq // 64), -(-Sk // 64)
    m = (rng.random((B, H, nbq, nbk)) < density).astype(np.uint8)
    return q, k, v, m


def _gpu(q, k, v, m, causal):
    return gpu_bf16_to_f64(bsa.bsattn_fwd_chunk(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v),
                                                to_gpu(m), causal))


def _oracle(q, k, v, m, causal):
    f = gen.bf16_bits_to_f64
    return oa.prefill(f(q), f(k), f(v), m, causal)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Sk", [(64, 256), (128, 448), (100, 300), (1, 130), (200, 201),
                                   (65, 4000), (256, 256)])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_every_element(Sq, Sk, D, causal):
    q, k, v, m = _case(2, 3, Sq, Sk, D, Sq * 31 + Sk + D)
    say(f"[prefill-chunk] Sq={Sq} Sk={Sk} D={D} causal={causal} blocks={int(m.sum())}")
    check_close(_gpu(q, k, v, m, causal), _oracle(q, k, v, m, causal),
                f"chunk Sq{Sq} Sk{Sk} D{D} c{causal}")


@pytest.mark.parametrize("D", [64, 128])
def test_chunk_dense_and_empty_rows(D):
    # dense mask: every causal key; empty mask rows: output 0
    q, k, v, _ = _case(1, 2, 192, 700, D, 5 + D)
    nbq, nbk = 3, 11
    m = np.ones((1, 2, nbq, nbk), np.uint8)
    m[0, 1, 1, :] = 0
    say(f"[prefill-chunk] dense + empty row D={D}")
    got = _gpu(q, k, v, m, True)
    check_close(got, _oracle(q, k, v, m, True), f"chunk dense D{D}")
    assert (got[0, 1, 64:128] == 0).all()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sk", [16384, 16448, 20000])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_long_rows(Sk, D, causal):
    """Mask rows of 256, 257 and 313 key blocks (the list walks up to four
    64-column words; longer rows take another path): a few columns scattered
    over the row, some rows whose only columns lie in the last words."""
    Sq = 192
    q, k, v, m = _case(1, 2, Sq, Sk, D, Sk + D + causal, density=0.03)
    nbk = m.shape[-1]
    m[0, 0, 0, :] = 0
    m[0, 0, 0, [63, 64, 191, 192, nbk - 1]] = 1        # word edges and the last column
    m[0, 1, 1, :] = 0
    m[0, 1, 1, nbk - 3:] = 1                           # only the row's last columns
    m[0, 1, 2, :] = 0
    m[0, 1, 2, [0, 255]] = 1
    say(f"[prefill-chunk] long rows Sq={Sq} Sk={Sk} nbk={nbk} D={D} causal={causal} blocks={int(m.sum())}")
    check_close(_gpu(q, k, v, m, causal), _oracle(q, k, v, m, causal),
                f"chunk long rows Sk{Sk} D{D} c{causal}")


def test_square_chunk_is_the_square_forward_bitwise():
    cfg = gen.CONFIGS["C1"]
    inp = gen.prefill_inputs(cfg, 0)
    m = om.build_mask_topk(inp["scores"], cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    a = bsa.bsattn_fwd(q, k, v, to_gpu(m), True)
    b = bsa.bsattn_fwd_chunk(q, k, v, to_gpu(m), True)
    say("[prefill-chunk] Sq = Sk vs bsattn_fwd")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_chunk_large_sampled_rows():
    """A 2048-query chunk at the end of a 16384-token context, D 128, top-k
    mask rows: sampled rows against the oracle computed row by row."""
    B, H, Sq, Sk, D = 1, 8, 2048, 16384, 128
    rng = np.random.default_rng(77)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sq, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, H, Sk, D), dtype=np.float32))
    nbq, nbk = Sq // 64, Sk // 64
    scores = rng.standard_normal((B, H, nbq, nbk), dtype=np.float32)
    top = np.argsort(-scores, axis=-1, kind="stable")[..., :24]
    m = np.zeros((B, H, nbq, nbk), np.uint8)
    np.put_along_axis(m, top, 1, axis=-1)
    past_blocks = (Sk - Sq) // 64
    m[..., np.arange(nbq), past_blocks + np.arange(nbq)] = 1   # each row's diagonal block
    say(f"[prefill-chunk] large Sq={Sq} Sk={Sk} blocks={int(m.sum())}")
    got = _gpu(q, k, v, m, True)
    f = gen.bf16_bits_to_f64
    rows = sorted({0, 1, 63, 64, 65, 1023, 2047} | set(rng.integers(0, Sq, 5).tolist()))
    for h in (0, 5):
        want = oa.prefill_head_rows(f(q[0, h]), f(k[0, h]), f(v[0, h]), m[0, h], True, rows)
        check_close(got[0, h, rows], want, f"large chunk h{h}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_longest_key_range(D, ragged, causal):
    """The longest key range the forward takes (bsattn_fwd_max_key_blocks:
    64511 key blocks at D 64, 48127 at D 128, about 4.1 M and 3.1 M tokens),
    one 64-query chunk at its end.  Every key block the mask leaves out holds
    NaN on the device, so a read of any of them into the result shows up as
    a non-finite output.  The expected rows come from the oracle on the
    selected blocks alone, laid end to end: every selected block before the
    last two is fully visible to every query row in both problems, and the
    last two (always selected) keep their offsets from the end of the keys,
    so each row sees the same keys at the same causal positions."""
    nbk = bsa.bsattn_fwd_max_key_blocks(D)
    assert nbk > 0
    Sk = nbk * 64 - (13 if ragged else 0)
    Sq, H = 64, 2
    rng = np.random.default_rng(nbk + 2 * ragged + causal)
    fixed = [{0, 1, 63, 64, 255, 256, 4095, 4096, nbk // 2, nbk - 66, nbk - 65, nbk - 64},
             {0}]
    sel = []
    for h in range(H):
        s = set(fixed[h]) | {nbk - 2, nbk - 1}
        if h == 0:
            s |= set(rng.integers(0, nbk - 2, 20).tolist())
        sel.append(sorted(s))
    q = gen.f32_to_bf16_bits(rng.standard_normal((1, H, Sq, D), dtype=np.float32))
    nan = float("nan")
    k_dev = torch.full((1, H, Sk, D), nan, dtype=torch.bfloat16, device="cuda")
    v_dev = torch.full((1, H, Sk, D), nan, dtype=torch.bfloat16, device="cuda")
    m = np.zeros((1, H, 1, nbk), np.uint8)
    kc, vc = [], []   # per head: the selected blocks' rows laid end to end
    for h in range(H):
        m[0, h, 0, sel[h]] = 1
        n_rows = sum(min(64, Sk - 64 * j) for j in sel[h])
        kh = gen.f32_to_bf16_bits(rng.standard_normal((n_rows, D), dtype=np.float32))
        vh = gen.f32_to_bf16_bits(rng.standard_normal((n_rows, D), dtype=np.float32))
        pos = 0
        for j in sel[h]:
            n = min(64, Sk - 64 * j)
            k_dev[0, h, 64 * j:64 * j + n] = to_gpu_bf16(kh[pos:pos + n])
            v_dev[0, h, 64 * j:64 * j + n] = to_gpu_bf16(vh[pos:pos + n])
            pos += n
        kc.append(kh)
        vc.append(vh)
    say(f"[prefill-chunk] longest key range D={D} nbk={nbk} Sk={Sk} causal={causal} "
        f"blocks={[len(s) for s in sel]}")
    got = gpu_bf16_to_f64(bsa.bsattn_fwd_chunk(to_gpu_bf16(q), k_dev, v_dev, to_gpu(m), causal))
    del k_dev, v_dev
    torch.cuda.empty_cache()
    f = gen.bf16_bits_to_f64
    for h in range(H):
        ones = np.ones((1, len(sel[h])), np.uint8)
        want = oa.prefill_head_rows(f(q[0, h]), f(kc[h]), f(vc[h]), ones, causal)
        check_close(got[0, h], want, f"longest key range D{D} ragged{ragged} c{causal} h{h}")
