"""GPU parity: mask-form and paged-KV sparse GQA decode against the float64 oracle."""
import functools

import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _base(name, seed):
    return gen.decode_inputs(gen.CONFIGS[name], seed)


def _f64(x):
    return gen.bf16_bits_to_f64(x)


def _mask_gpu(inp, ns, bm=None):
    q, k, v = (to_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    bm = inp["block_mask"] if bm is None else bm
    return gpu_bf16_to_f64(bsa.bsattn_decode_gqa_mask(q, k, v, to_gpu(inp["cu_seqlens_k"]),
                                                      to_gpu(bm), num_splits=ns))


def _mask_oracle(inp, bm=None):
    bm = inp["block_mask"] if bm is None else bm
    return oa.decode_gqa_mask(_f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"]), inp["cu_seqlens_k"], bm)


def _paged_gpu(inp, ns, table=None, idx=None):
    table = inp["block_table"] if table is None else table
    idx = inp["block_indices"] if idx is None else idx
    out = bsa.bsattn_decode_gqa_paged(
        to_gpu_bf16(inp["q"]), to_gpu_bf16(inp["k_cache"]), to_gpu_bf16(inp["v_cache"]),
        to_gpu(inp["cache_seqlens"]), to_gpu(table), to_gpu(idx), num_splits=ns)
    return gpu_bf16_to_f64(out)


def _paged_oracle(inp, table=None, idx=None):
    table = inp["block_table"] if table is None else table
    idx = inp["block_indices"] if idx is None else idx
    return oa.decode_gqa_paged(_f64(inp["q"]), _f64(inp["k_cache"]), _f64(inp["v_cache"]),
                               inp["cache_seqlens"], table, idx)


@pytest.mark.parametrize("name", ["P2", "C5"])
def test_mask_form_configs(name):
    cfg = gen.CONFIGS[name]
    inp = gen.decode_mask_inputs(cfg, 0, base=_base(name, 0))
    want = _mask_oracle(inp)
    nbk = inp["block_mask"].shape[2]
    for ns in (0, 1, 5):
        say(f"[decode-mask] {name} num_blocks={nbk} ns={ns}")
        check_close(_mask_gpu(inp, ns), want, f"mask {name} ns={ns}")
    # the index form over the same selection gives the same attention
    idx_out = gpu_bf16_to_f64(bsa.bsattn_decode_gqa(
        *(to_gpu_bf16(inp[n]) for n in ("q", "k", "v")), to_gpu(inp["cu_seqlens_k"]),
        to_gpu(inp["block_indices"])))
    assert np.abs(idx_out - want).max() <= 1e-2


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_mask_form_ragged(D, G):
    rng = np.random.default_rng(100 + D + G)
    lens = np.array([1, 63, 64, 65, 200, 1000])
    B, Hkv = len(lens), 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    nbk = 20                                       # columns past every sequence's end
    bm = (rng.random((B, Hkv, nbk)) < 0.35).astype(np.uint8)
    bm[0, 0, :] = 0                                # nothing selected
    inp = {"cu_seqlens_k": cu, "block_mask": bm,
           "q": gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv * G, D), dtype=np.float32)),
           "k": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32)),
           "v": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))}
    want = _mask_oracle(inp)
    for ns in (1, 3, nbk):
        say(f"[decode-mask] ragged D={D} G={G} ns={ns}")
        got = _mask_gpu(inp, ns)
        check_close(got, want, f"mask D{D} G{G} ns{ns}")
        assert (got[0, :G] == 0).all()


@pytest.mark.parametrize("page_size", [64, 256])
@pytest.mark.parametrize("name", ["P2", "C5"])
def test_paged_configs(name, page_size):
    cfg = gen.CONFIGS[name]
    inp = gen.decode_paged_inputs(cfg, 0, page_size=page_size, base=_base(name, 0))
    want = _paged_oracle(inp)
    for ns in (0, 1, 7):
        say(f"[decode-paged] {name} page={page_size} pages={inp['k_cache'].shape[0]} ns={ns}")
        check_close(_paged_gpu(inp, ns), want, f"paged {name} p{page_size} ns={ns}")


@pytest.mark.parametrize("D", [64, 128])
def test_paged_ragged_and_bad_entries(D):
    cfg = gen.DecodeConfig("paged_ragged", B=4, Hq=8, Hkv=2, D=D, len_lo=1, len_hi=700,
                           max_selected_blocks=9, sparse_ratio=0.5)
    inp = gen.decode_paged_inputs(cfg, 3, page_size=128, spare_pages=5)
    want = _paged_oracle(inp)
    say(f"[decode-paged] ragged D={D} lens={inp['cache_seqlens'].tolist()}")
    check_close(_paged_gpu(inp, 2), want, f"paged ragged D{D}")
    # table entries outside the cache, a missing table column and a negative length
    table = inp["block_table"].copy()
    table[0, 0] = inp["k_cache"].shape[0] + 3
    table[1, 0] = -2
    idx = inp["block_indices"].copy()
    idx[2, 0, 0] = table.shape[1] * 2 + 1          # logical page past the table
    want2 = _paged_oracle(inp, table, idx)
    say(f"[decode-paged] bad entries D={D}")
    check_close(_paged_gpu(inp, 3, table, idx), want2, f"paged bad entries D{D}")
    seqlens = inp["cache_seqlens"].copy()
    seqlens[3] = -5
    out = bsa.bsattn_decode_gqa_paged(
        to_gpu_bf16(inp["q"]), to_gpu_bf16(inp["k_cache"]), to_gpu_bf16(inp["v_cache"]),
        to_gpu(seqlens), to_gpu(inp["block_table"]), to_gpu(inp["block_indices"]), num_splits=2)
    got = gpu_bf16_to_f64(out)
    assert (got[3] == 0).all()
    np.testing.assert_array_equal(got[:3], _paged_gpu(inp, 2)[:3])


def test_paged_identity_table_matches_packed_bitwise():
    """Pages laid out in sequence order with page_size = 64 put every block at
    the packed layout's relative position: the same kernel arithmetic runs, so
    the output is bit-identical to the packed index form."""
    cfg = gen.CONFIGS["P2"]
    inp = _base("P2", 1)
    lens = inp["lens"]
    B, Hkv, D = cfg.B, cfg.Hkv, cfg.D
    per = [-(-int(x) // 64) for x in lens]
    kc = np.zeros((sum(per), 64, Hkv, D), np.uint16)
    vc = np.zeros_like(kc)
    table = np.full((B, max(per)), -1, np.int32)
    p = 0
    for b in range(B):
        for lp in range(per[b]):
            t0, t1 = lp * 64, min(lp * 64 + 64, int(lens[b]))
            c0 = int(inp["cu_seqlens_k"][b])
            kc[p, :t1 - t0] = inp["k"][c0 + t0:c0 + t1]
            vc[p, :t1 - t0] = inp["v"][c0 + t0:c0 + t1]
            table[b, lp] = p
            p += 1
    q = to_gpu_bf16(inp["q"])
    paged = bsa.bsattn_decode_gqa_paged(q, to_gpu_bf16(kc), to_gpu_bf16(vc),
                                        to_gpu(lens.astype(np.int32)), to_gpu(table),
                                        to_gpu(inp["block_indices"]), num_splits=3)
    packed = bsa.bsattn_decode_gqa(q, to_gpu_bf16(inp["k"]), to_gpu_bf16(inp["v"]),
                                   to_gpu(inp["cu_seqlens_k"]), to_gpu(inp["block_indices"]),
                                   num_splits=3)
    say("[decode-paged] identity table vs packed")
    assert torch.equal(paged.view(torch.int16), packed.view(torch.int16))
