"""GPU: tensors past 4 GiB, so every address above 2^32 bytes must be formed
in 64 bits.  Only the selected blocks hold data; every other K/V row is NaN on
the device (a read of one would make the output non-finite), and the host
side keeps just the selected rows.  The expected values come from the oracle
on the selected blocks laid end to end, which leaves every row's visible keys
and their causal positions unchanged (the reasoning is given per test).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from oracle import attention as oa
from tests.gpu_util import check_close, gpu_bf16_to_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def test_chunk_forward_heads_past_4gib():
    """One 64-query chunk at the end of the longest key range at D 128, eight
    heads: K and V are 6.3 GB each, so heads 6 and 7 start past 4 GiB.  The
    last two key blocks are always selected, so laying the selected blocks
    end to end keeps the causal relation of every row (as in the chunk
    tests' longest-range case)."""
    D, H = 128, 8
    nbk = bsa.bsattn_fwd_max_key_blocks(D)
    Sk, Sq = nbk * 64 - 5, 64
    assert H * Sk * D * 2 > 4 * GIB
    rng = np.random.default_rng(4242)
    sel = [sorted(set(rng.integers(0, nbk - 2, 12).tolist()) | {0, nbk - 2, nbk - 1}) for _ in range(H)]
    q = gen.f32_to_bf16_bits(rng.standard_normal((1, H, Sq, D), dtype=np.float32))
    nan = float("nan")
    k_dev = torch.full((1, H, Sk, D), nan, dtype=torch.bfloat16, device="cuda")
    v_dev = torch.full((1, H, Sk, D), nan, dtype=torch.bfloat16, device="cuda")
    m = np.zeros((1, H, 1, nbk), np.uint8)
    kc, vc = [], []
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
    say(f"[large-offsets] chunk forward H={H} Sk={Sk} D={D}: K/V {k_dev.numel() * 2 / GIB:.2f} GiB each")
    got = gpu_bf16_to_f64(bsa.bsattn_fwd_chunk(to_gpu_bf16(q), k_dev, v_dev, to_gpu(m), True))
    del k_dev, v_dev
    torch.cuda.empty_cache()
    f = gen.bf16_bits_to_f64
    for h in range(H):
        want = oa.prefill_head_rows(f(q[0, h]), f(kc[h]), f(vc[h]), np.ones((1, len(sel[h])), np.uint8), True)
        check_close(got[0, h], want, f"chunk forward past 4 GiB h{h}")


@pytest.mark.parametrize("form", ["index", "mask"])
def test_decode_sequences_past_4gib(form):
    """Three sequences of about two million tokens, eight KV heads, D 128:
    packed K and V are 12.3 GB each, so the last sequence starts past 8 GiB.
    The expected values come from the oracle on a packed problem that keeps,
    per sequence, only the blocks some KV head selects, in order, with the
    sequence's last (partial) block still last: each query head then sees the
    same tokens."""
    B, Hq, Hkv, D = 3, 32, 8, 128
    lens = np.array([2_000_003, 2_000_064, 1_999_937])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    assert T * Hkv * D * 2 > 8 * GIB
    rng = np.random.default_rng(777)
    ms = 24
    idx = np.full((B, Hkv, ms), -1, np.int32)
    for b in range(B):
        nbb = -(-int(lens[b]) // 64)
        for h in range(Hkv):
            s = sorted(set(rng.integers(0, nbb - 1, 20).tolist()) | {nbb - 1})[::-1]
            idx[b, h, :len(s)] = s
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
    nan = float("nan")
    k_dev = torch.full((T, Hkv, D), nan, dtype=torch.bfloat16, device="cuda")
    v_dev = torch.full((T, Hkv, D), nan, dtype=torch.bfloat16, device="cuda")
    # the compact problem: per sequence, the union of the selected blocks
    k_parts, v_parts, cu_c, idx_c = [], [], [0], np.full((B, Hkv, ms), -1, np.int32)
    for b in range(B):
        L = int(lens[b])
        union = sorted({int(j) for j in idx[b].ravel() if j >= 0})
        n_rows = sum(min(64, L - 64 * j) for j in union)
        kb = gen.f32_to_bf16_bits(rng.standard_normal((n_rows, Hkv, D), dtype=np.float32))
        vb = gen.f32_to_bf16_bits(rng.standard_normal((n_rows, Hkv, D), dtype=np.float32))
        pos, where = 0, {}
        for p, j in enumerate(union):
            n = min(64, L - 64 * j)
            where[j] = p
            for h in range(Hkv):
                if j in idx[b, h]:
                    r0 = int(cu[b]) + 64 * j
                    k_dev[r0:r0 + n, h] = to_gpu_bf16(kb[pos:pos + n, h])
                    v_dev[r0:r0 + n, h] = to_gpu_bf16(vb[pos:pos + n, h])
            pos += n
        k_parts.append(kb)
        v_parts.append(vb)
        cu_c.append(cu_c[-1] + n_rows)
        for h in range(Hkv):
            row = [where[int(j)] for j in idx[b, h] if j >= 0]
            idx_c[b, h, :len(row)] = row
    cu_c = np.array(cu_c, np.int32)
    f = gen.bf16_bits_to_f64
    want = oa.decode_gqa(f(q), f(np.concatenate(k_parts)), f(np.concatenate(v_parts)), cu_c, idx_c)
    say(f"[large-offsets] decode {form} total_k={T}: K/V {k_dev.numel() * 2 / GIB:.2f} GiB each")
    qd, cud = to_gpu_bf16(q), to_gpu(cu)
    for ns in (1, 4):
        if form == "index":
            out = bsa.bsattn_decode_gqa(qd, k_dev, v_dev, cud, to_gpu(idx), num_splits=ns)
        else:
            nbk = max(-(-int(x) // 64) for x in lens)
            bm = np.zeros((B, Hkv, nbk), np.uint8)
            for b in range(B):
                for h in range(Hkv):
                    bm[b, h, idx[b, h][idx[b, h] >= 0]] = 1
            out = bsa.bsattn_decode_gqa_mask(qd, k_dev, v_dev, cud, to_gpu(bm), num_splits=ns)
        check_close(gpu_bf16_to_f64(out), want, f"decode {form} past 4 GiB ns{ns}")
    del k_dev, v_dev
    torch.cuda.empty_cache()


def test_square_forward_heads_past_4gib():
    """bsattn_fwd on B1 H80 S262144 D128: q, k, v and out are 5 GiB each and
    the last heads start past 4 GiB (the long-row split's workspace would
    pass 2 GiB, so rows run whole).  A few work items of heads 0, 40 and 79
    select scattered blocks and are checked against the oracle; every other
    item selects key block 0 only with q = 0, so its rows are the mean of
    block 0's values (a closed form).  K/V rows no item selects are NaN."""
    B, H, S, D = 1, 80, 262144, 128
    nb = S // 64
    assert H * S * D * 2 > 4 * GIB
    rng = np.random.default_rng(99)
    heads, qblocks = (0, 40, 79), (1, 2, 2047, nb - 2, nb - 1)
    m = np.zeros((B, H, nb, nb), np.uint8)
    m[0, :, :, 0] = 1
    sel = {}
    for h in heads:
        for i in qblocks:
            s = sorted(set(rng.integers(0, i + 1, 8).tolist()) | {0, i})
            m[0, h, i, :] = 0
            m[0, h, i, s] = 1
            sel[h, i] = s
    nan = float("nan")
    q_dev = torch.zeros((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    k_dev = torch.full((B, H, S, D), nan, dtype=torch.bfloat16, device="cuda")
    v_dev = torch.full((B, H, S, D), nan, dtype=torch.bfloat16, device="cuda")
    k0 = gen.f32_to_bf16_bits(rng.standard_normal((H, 64, D), dtype=np.float32))
    v0 = gen.f32_to_bf16_bits(rng.standard_normal((H, 64, D), dtype=np.float32))
    k_dev[0, :, :64] = to_gpu_bf16(k0)
    v_dev[0, :, :64] = to_gpu_bf16(v0)
    host = {}
    for h in heads:   # host copies: zeros where the device holds NaN (never weighted)
        qh = np.zeros((S, D), np.uint16)
        kh = np.zeros((S, D), np.uint16)
        vh = np.zeros((S, D), np.uint16)
        kh[:64], vh[:64] = k0[h], v0[h]
        blocks = sorted({j for i in qblocks for j in sel[h, i]} - {0})
        for j in blocks:
            kh[64 * j:64 * j + 64] = gen.f32_to_bf16_bits(rng.standard_normal((64, D), dtype=np.float32))
            vh[64 * j:64 * j + 64] = gen.f32_to_bf16_bits(rng.standard_normal((64, D), dtype=np.float32))
            k_dev[0, h, 64 * j:64 * j + 64] = to_gpu_bf16(kh[64 * j:64 * j + 64])
            v_dev[0, h, 64 * j:64 * j + 64] = to_gpu_bf16(vh[64 * j:64 * j + 64])
        for i in qblocks:
            qh[64 * i:64 * i + 64] = gen.f32_to_bf16_bits(rng.standard_normal((64, D), dtype=np.float32))
            q_dev[0, h, 64 * i:64 * i + 64] = to_gpu_bf16(qh[64 * i:64 * i + 64])
        host[h] = (qh, kh, vh)
    assert bsa.bsattn_fwd_workspace_bytes(B, H, S, D) == 0
    say(f"[large-offsets] square forward B{B} H{H} S{S} D{D}: q/k/v/out {q_dev.numel() * 2 / GIB:.2f} GiB each")
    out = bsa.bsattn_fwd(q_dev, k_dev, v_dev, to_gpu(m), True)
    f = gen.bf16_bits_to_f64
    for h in heads:
        qh, kh, vh = host[h]
        rows = np.array([64 * i + r for i in qblocks for r in (0, 31, 63)])
        got = gpu_bf16_to_f64(out[0, h, torch.from_numpy(rows).cuda()])
        want = oa.prefill_head_rows(f(qh), f(kh), f(vh), m[0, h], True, rows)
        check_close(got, want, f"square forward past 4 GiB h{h}")
    # items that see block 0 only, with q = 0: every visible key weighs the same
    for h in (1, 41, 78, 79):
        for i in (5, 3000, nb - 1):
            if (h, i) in sel:
                continue
            got = gpu_bf16_to_f64(out[0, h, 64 * i:64 * i + 64])
            want = np.broadcast_to(f(v0[h]).mean(axis=0), got.shape)
            check_close(got, want, f"square forward past 4 GiB, block 0 only, h{h} i{i}")
    del q_dev, k_dev, v_dev, out
    torch.cuda.empty_cache()


def test_paged_decode_cache_past_4gib():
    """Paged decode over a 10 000-page cache (256-token pages, eight KV
    heads, D 128: K and V caches of 4.9 GiB each), pages handed out in a
    shuffled order so blocks sit anywhere in the cache.  Expected values: the
    oracle's packed decode on the union of the selected blocks, laid end to
    end per sequence with the last (partial) block still last, as in the
    packed test above."""
    B, Hq, Hkv, D, ps = 2, 32, 8, 128, 256
    lens = np.array([1_000_037, 999_999])
    per_seq = [-(-int(x) // ps) for x in lens]
    num_pages = 10_000
    assert num_pages * ps * Hkv * D * 2 > 4 * GIB and sum(per_seq) < num_pages
    rng = np.random.default_rng(31337)
    perm = rng.permutation(num_pages)
    table = np.full((B, max(per_seq)), -1, np.int32)
    p = 0
    for b in range(B):
        table[b, :per_seq[b]] = perm[p:p + per_seq[b]]
        p += per_seq[b]
    ms = 24
    idx = np.full((B, Hkv, ms), -1, np.int32)
    for b in range(B):
        nbb = -(-int(lens[b]) // 64)
        for h in range(Hkv):
            s = sorted(set(rng.integers(0, nbb - 1, 20).tolist()) | {nbb - 1})[::-1]
            idx[b, h, :len(s)] = s
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
    nan = float("nan")
    kc = torch.full((num_pages, ps, Hkv, D), nan, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((num_pages, ps, Hkv, D), nan, dtype=torch.bfloat16, device="cuda")
    k_parts, v_parts, cu_c, idx_c = [], [], [0], np.full((B, Hkv, ms), -1, np.int32)
    for b in range(B):
        L = int(lens[b])
        union = sorted({int(j) for j in idx[b].ravel() if j >= 0})
        n_rows = sum(min(64, L - 64 * j) for j in union)
        kb = gen.f32_to_bf16_bits(rng.standard_normal((n_rows, Hkv, D), dtype=np.float32))
        vb = gen.f32_to_bf16_bits(rng.standard_normal((n_rows, Hkv, D), dtype=np.float32))
        pos, where = 0, {}
        for pidx, j in enumerate(union):
            n = min(64, L - 64 * j)
            where[j] = pidx
            page, r0 = int(table[b, (64 * j) // ps]), (64 * j) % ps
            for h in range(Hkv):
                if j in idx[b, h]:
                    kc[page, r0:r0 + n, h] = to_gpu_bf16(kb[pos:pos + n, h])
                    vc[page, r0:r0 + n, h] = to_gpu_bf16(vb[pos:pos + n, h])
            pos += n
        k_parts.append(kb)
        v_parts.append(vb)
        cu_c.append(cu_c[-1] + n_rows)
        for h in range(Hkv):
            row = [where[int(j)] for j in idx[b, h] if j >= 0]
            idx_c[b, h, :len(row)] = row
    f = gen.bf16_bits_to_f64
    want = oa.decode_gqa(f(q), f(np.concatenate(k_parts)), f(np.concatenate(v_parts)),
                         np.array(cu_c, np.int32), idx_c)
    say(f"[large-offsets] paged decode {num_pages} pages: caches {kc.numel() * 2 / GIB:.2f} GiB each")
    for ns in (1, 4):
        out = bsa.bsattn_decode_gqa_paged(to_gpu_bf16(q), kc, vc, to_gpu(lens.astype(np.int32)),
                                          to_gpu(table), to_gpu(idx), num_splits=ns)
        check_close(gpu_bf16_to_f64(out), want, f"paged decode past 4 GiB ns{ns}")
    del kc, vc
    torch.cuda.empty_cache()


def test_xattn_estimate_heads_past_4gib():
    """The whole estimate at stride 8 on B1 H270 S65536 D128 (the longest key
    range the block sums and the selection take): q and k are 4.2 GiB each
    and the log-sum workspace 8.4 GiB, so the last heads' operands and
    log-sums sit past 4 GiB.  Heads 0 and 269 hold seeded N(0, 1) data and
    head 268 zeros (a uniform softmax); all three are checked against the
    oracle, and their selections are checked valid for the oracle's sums."""
    from tests.gpu_util import parallel_map
    from tests.test_gpu_xattn import SUM_ATOL, SUM_RTOL, _check_valid_selection
    from oracle import xattn as ox

    B, H, S, D, stride = 1, 270, 65536, 128, 8
    assert H * S * D * 2 > 4 * GIB
    rng = np.random.default_rng(2718)
    q_dev = torch.zeros((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    k_dev = torch.zeros((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    host = {}
    for h in (0, 269):
        qh = gen.f32_to_bf16_bits(rng.standard_normal((S, D), dtype=np.float32))
        kh = gen.f32_to_bf16_bits(rng.standard_normal((S, D), dtype=np.float32))
        q_dev[0, h] = to_gpu_bf16(qh)
        k_dev[0, h] = to_gpu_bf16(kh)
        host[h] = (qh, kh)
    host[268] = (np.zeros((S, D), np.uint16), np.zeros((S, D), np.uint16))
    say(f"[large-offsets] xattn estimate B{B} H{H} S{S} D{D}: q/k {q_dev.numel() * 2 / GIB:.2f} GiB each")
    mask, sums = bsa.bsattn_xattn_estimate(q_dev, k_dev, stride, 1.0, 0.9, True, True, True,
                                           write_sums=True)
    heads = sorted(host)
    got_s = {h: sums[:, h:h + 1].cpu().numpy() for h in heads}
    got_m = {h: mask[:, h:h + 1].cpu().numpy() for h in heads}
    del q_dev, k_dev, mask, sums
    torch.cuda.empty_cache()
    f = gen.bf16_bits_to_f64
    wants = parallel_map(lambda h: ox.block_sums(f(host[h][0])[None, None], f(host[h][1])[None, None],
                                                 stride, 1.0, True), heads, workers=3)
    tol = 1024 * (SUM_ATOL + SUM_RTOL * 8)
    for h, want in zip(heads, wants):
        np.testing.assert_allclose(got_s[h], want, rtol=SUM_RTOL, atol=SUM_ATOL)
        _check_valid_selection(got_m[h], want, 0.9, True, True, True, tol)
        say(f"  head {h}: block sums and selection ok")
