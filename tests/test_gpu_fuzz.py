"""GPU parity over seeded random shapes: every form of the hot path against
the float64 oracle, on shapes drawn from a fixed generator (so every run
checks the same cases) rather than picked by hand: batch and head counts,
ragged lengths, head dims, causal or not, mask density, split counts, group
sizes and page sizes.  Each case prints what it is before it runs.  Outputs
meet the stated tolerance (max-abs 1e-2, mean-abs 1e-3) at the workloads'
logit scales; one extra set of prefill cases at sharper logits is held to
the guide's own relative bound instead (check_guide)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from oracle import mask as om
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

CASES = 12


def check_guide(got, want, what):
    """The block-sparse guide's own reference check (§5: assert_close with
    atol = rtol = 1e-2, elementwise |got - want| <= 1e-2 + 1e-2 |want|), plus
    the mean absolute error bound.  Used only past the workloads' logit
    scales (q and k at 3x N(0,1), D = 128: logits with a standard deviation
    near 9), where a sharply peaked softmax makes outputs copies of single V
    values, some of magnitude 4 or more; bfloat16 numbers there are 1/32
    apart, so storing the output alone can be off by up to 1/64 > 1e-2 (the
    worst case measured: 4.2654 stored as 4.25, with the value before the
    store within 4e-5 of the oracle)."""
    assert got.shape == want.shape and np.isfinite(got).all(), what
    err = np.abs(got - want)
    bound = 1e-2 + 1e-2 * np.abs(want)
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {what}: max_abs={err.max() if err.size else 0:.3e} mean_abs={err.mean() if err.size else 0:.3e} "
        f"max err/bound={worst:.3f}")
    assert worst <= 1.0, f"{what}: error {worst:.3f}x the guide's bound"
    assert (err.mean() if err.size else 0.0) <= 1e-3, f"{what}: mean abs err {err.mean()}"


def _bits(rng, shape, scale=1.0):
    return gen.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * scale)


def _prefill_case(rng, scales):
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    D = int(rng.choice([64, 128]))
    Sk = int(rng.integers(1, 1500))
    Sq = Sk if rng.random() < 0.5 else int(rng.integers(1, Sk + 1))
    causal = bool(rng.random() < 0.7)
    nbq, nbk = -(-Sq // 64), -(-Sk // 64)
    density = float(rng.choice([0.0, 0.1, 0.5, 1.0]))
    mask = (rng.random((B, H, nbq, nbk)) < density).astype(np.uint8)
    scale = float(rng.choice(scales))
    q, k, v = _bits(rng, (B, H, Sq, D), scale), _bits(rng, (B, H, Sk, D), scale), _bits(rng, (B, H, Sk, D))
    say(f"[fuzz-prefill] B{B} H{H} Sq{Sq} Sk{Sk} D{D} causal={causal} density={density} scale={scale}")
    qg, kg, vg, mg = to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), to_gpu(mask)
    if Sq == Sk:
        got = gpu_bf16_to_f64(bsa.bsattn_fwd(qg, kg, vg, mg, causal))
        idx, cnt = bsa.bsattn_mask_to_indices(mg, causal)
        via_list = bsa.bsattn_fwd_indices(qg, kg, vg, idx, cnt, causal)
        assert np.array_equal(gpu_bf16_to_f64(via_list), got)
    else:
        got = gpu_bf16_to_f64(bsa.bsattn_fwd_chunk(qg, kg, vg, mg, causal))
    f = gen.bf16_bits_to_f64
    return got, oa.prefill(f(q), f(k), f(v), mask, causal)


@pytest.mark.parametrize("case", range(CASES))
def test_prefill_random_shapes(case):
    """q and k at 0.3 to 1x N(0,1), the workloads' range: the stated tolerance."""
    got, want = _prefill_case(np.random.default_rng(1000 + case), [0.3, 0.5, 1.0])
    check_close(got, want, f"fuzz prefill {case}")


@pytest.mark.parametrize("case", range(4))
def test_prefill_sharp_logits_within_the_guides_bound(case):
    """q and k at 3x N(0,1): the guide's relative bound (see check_guide)."""
    rng = np.random.default_rng(1500 + case)
    got, want = _prefill_case(rng, [3.0])
    check_guide(got, want, f"fuzz prefill, sharp logits {case}")


@pytest.mark.parametrize("case", range(CASES))
def test_fused_random_shapes(case):
    rng = np.random.default_rng(2000 + case)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    S = int(rng.integers(1, 1200))
    nb = -(-S // 64)
    causal = bool(rng.random() < 0.7)
    dense2, diag = bool(rng.random() < 0.5), bool(rng.random() < 0.7)
    scores = rng.standard_normal((B, H, nb, nb)).astype(np.float32)
    if rng.random() < 0.3:
        scores = np.round(scores * 2) / 2   # ties
    q, k, v = (_bits(rng, (B, H, S, D)) for _ in range(3))
    qg, kg, vg, sg = to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), to_gpu(scores)
    if rng.random() < 0.5:
        topk = int(rng.integers(0, nb + 1))
        say(f"[fuzz-fused {case}] topk={topk} B{B} H{H} S{S} D{D} causal={causal} dense2={dense2} diag={diag}")
        out, m = bsa.bsattn_fwd_topk(qg, kg, vg, sg, topk, dense2, diag, causal, write_mask=True)
        want_mask = om.build_mask_topk(scores, topk, dense2, diag)
    else:
        thr = float(rng.choice([-0.5, 0.0, 0.7, 2.0]))
        say(f"[fuzz-fused {case}] threshold={thr} B{B} H{H} S{S} D{D} causal={causal} dense2={dense2} diag={diag}")
        out, m = bsa.bsattn_fwd_threshold(qg, kg, vg, sg, thr, dense2, diag, causal, write_mask=True)
        want_mask = om.build_mask_threshold(scores, thr, dense2, diag)
    np.testing.assert_array_equal(m.cpu().numpy(), want_mask)
    f = gen.bf16_bits_to_f64
    check_close(gpu_bf16_to_f64(out), oa.prefill(f(q), f(k), f(v), want_mask, causal),
                f"fuzz fused {case}")


@pytest.mark.parametrize("case", range(CASES))
def test_decode_random_shapes(case):
    rng = np.random.default_rng(3000 + case)
    B = int(rng.integers(1, 6))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 3, 8, 16, 20, 64]))
    Hq = Hkv * G
    D, Dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    lens = rng.integers(1, 3000, size=B)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    ms = int(rng.integers(1, 40))
    idx = np.full((B, Hkv, ms), -1, np.int32)
    for b in range(B):
        nbb = -(-int(lens[b]) // 64)
        for h in range(Hkv):
            n = int(rng.integers(0, min(ms, nbb) + 1))
            idx[b, h, :n] = rng.choice(nbb, n, replace=False)
            if rng.random() < 0.2:
                idx[b, h, rng.integers(0, ms)] = nbb + 3   # out of range: selects nothing
    q, k, v = _bits(rng, (B, Hq, D)), _bits(rng, (T, Hkv, D)), _bits(rng, (T, Hkv, Dv))
    ns = min(int(rng.choice([0, 1, 2, 5])), ms)
    form = str(rng.choice(["indices", "mask", "paged"]))
    say(f"[fuzz-decode {case}] {form} B{B} Hq{Hq} Hkv{Hkv} D{D} Dv{Dv} max_sel{ms} splits{ns} lens{list(lens)}")
    f = gen.bf16_bits_to_f64
    qg, kg, vg, cug = to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), to_gpu(cu)
    if form == "indices":
        got = bsa.bsattn_decode_gqa(qg, kg, vg, cug, to_gpu(idx), num_splits=ns)
        want = oa.decode_gqa(f(q), f(k), f(v), cu, idx)
    elif form == "mask":
        nbk = int(max(-(-int(x) // 64) for x in lens)) + int(rng.integers(0, 3))
        bm = np.zeros((B, Hkv, nbk), np.uint8)
        for b in range(B):
            for h in range(Hkv):
                sel = idx[b, h]
                sel = sel[(sel >= 0) & (sel < nbk)]
                bm[b, h, sel] = rng.integers(1, 256, size=sel.size)   # any nonzero byte selects
        got = bsa.bsattn_decode_gqa_mask(qg, kg, vg, cug, to_gpu(bm), num_splits=min(ns, nbk))
        want = oa.decode_gqa_mask(f(q), f(k), f(v), cu, bm)
    else:
        page = int(rng.choice([64, 128, 256]))
        per = [-(-int(x) // page) for x in lens]
        npg = sum(per) + 2
        perm = rng.permutation(npg)
        kc = _bits(rng, (npg, page, Hkv, D))
        vc = _bits(rng, (npg, page, Hkv, Dv))
        table = np.full((B, max(per)), -1, np.int32)
        p = 0
        for b in range(B):
            for lp in range(per[b]):
                pg = int(perm[p]); p += 1
                table[b, lp] = pg
                t0, t1 = lp * page, min((lp + 1) * page, int(lens[b]))
                kc[pg, :t1 - t0] = k[cu[b] + t0:cu[b] + t1]
                vc[pg, :t1 - t0] = v[cu[b] + t0:cu[b] + t1]
        got = bsa.bsattn_decode_gqa_paged(qg, to_gpu_bf16(kc), to_gpu_bf16(vc),
                                          to_gpu(lens.astype(np.int32)), to_gpu(table), to_gpu(idx),
                                          num_splits=ns)
        want = oa.decode_gqa_paged(f(q), f(kc), f(vc), lens.astype(np.int32), table, idx)
    check_close(gpu_bf16_to_f64(got), want, f"fuzz decode {case} ({form})")
