"""The decode entry point that allocates nothing (bsattn_decode_gqa_noalloc).

Called through the C ABI (the binding's ctypes call), its output must equal
bsattn_decode_gqa's with the same split count bit for bit — the same kernels
over the same data, only the partials live in the library's static scratch
array — and meet the oracle's tolerance.  Two calls in a row, the second on
a smaller input, check that nothing left in the shared scratch by the first
call leaks into the second.  A split count whose partials exceed the scratch
array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _dev_inputs(d):
    return (to_gpu_bf16(d["q"]), to_gpu_bf16(d["k"]), to_gpu_bf16(d["v"]),
            to_gpu(d["cu_seqlens_k"]), to_gpu(d["block_indices"]))


def _oracle(d):
    f = gen.bf16_bits_to_f64
    return oa.decode_gqa(f(d["q"]), f(d["k"]), f(d["v"]), d["cu_seqlens_k"], d["block_indices"])


def _ragged(seed, D, G):
    rng = np.random.default_rng(seed)
    lens = np.array([1, 65, 700, 130])
    B, Hkv = len(lens), 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    idx = np.full((B, Hkv, 6), -1, np.int32)
    for b, L in enumerate(lens):
        nbb = -(-int(L) // 64)
        for h in range(Hkv):
            n = int(rng.integers(1, min(nbb, 5) + 1))
            idx[b, h, :n] = rng.choice(nbb, size=n, replace=False)
    return {"cu_seqlens_k": cu, "block_indices": idx,
            "q": gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv * G, D), dtype=np.float32)),
            "k": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32)),
            "v": gen.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))}


def test_two_calls_in_a_row_match_the_workspace_form():
    big = gen.decode_inputs(gen.CONFIGS["C5"], 0)
    small = _ragged(3, 128, 4)
    assert bsa.bsattn_decode_noalloc_scratch_bytes() == 8 << 20
    for name, d, splits in (("C5", big, (0, 4, 16)), ("ragged", small, (3, 0, 1))):
        q, k, v, cu, idx = _dev_inputs(d)
        want = _oracle(d)
        for ns in splits:
            say(f"[no-alloc] {name} ns={ns}")
            ref = bsa.bsattn_decode_gqa(q, k, v, cu, idx, num_splits=ns)
            got = bsa.bsattn_decode_gqa_noalloc(q, k, v, cu, idx, num_splits=ns)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (name, ns)
            check_close(gpu_bf16_to_f64(got), want, f"no-alloc {name} ns={ns}")


def test_smaller_second_call_with_other_head_dim():
    a, b = _ragged(5, 128, 16), _ragged(6, 64, 1)
    for name, d in (("D128 G16", a), ("D64 G1", b)):
        q, k, v, cu, idx = _dev_inputs(d)
        say(f"[no-alloc] {name}")
        got = bsa.bsattn_decode_gqa_noalloc(q, k, v, cu, idx, num_splits=5)
        ref = bsa.bsattn_decode_gqa(q, k, v, cu, idx, num_splits=5)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name
        check_close(gpu_bf16_to_f64(got), _oracle(d), f"no-alloc {name}")


def test_too_large_for_the_scratch_is_refused():
    # B * Hq * splits partials of D floats beyond 8 MiB: 64 * 64 * 64 * 128 * 4 B = 128 MiB
    B, Hq, Hkv, D, ms = 64, 64, 4, 128, 64
    assert bsa.bsattn_decode_workspace_bytes(B, Hq, D, 64) > bsa.bsattn_decode_noalloc_scratch_bytes()
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, Hkv, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    idx = torch.full((B, Hkv, ms), -1, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), 3.0, dtype=torch.bfloat16, device="cuda")
    say("[no-alloc] oversized split count is refused")
    with pytest.raises(bsa.BsattnError) as e:
        bsa.bsattn_decode_gqa_noalloc(q, k, k, cu, idx, num_splits=64, out=out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert (out == 3.0).all()     # nothing was enqueued
