"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues only kernel launches (no memset, no copy, no host
synchronisation), so a captured call replays as the eager call runs.  Each
case captures one call sequence on static input buffers, then for several
rounds: new inputs go into the static buffers, unrelated eager work runs, the
graph replays, and its output must equal, bit for bit, the eager call on
those same inputs (the kernels are deterministic).  The split-row flags, the
decode partials and the estimator's log-sums are rewritten by every replay,
so nothing a previous replay left behind may leak into the next."""
import numpy as np
import pytest
import torch

import block_sparse_attention_amd as bsa
from block_sparse_attention_amd import inputs as gen
from tests.gpu_util import say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(run):
    """Warm `run` up on a side stream, then capture it; returns (graph, outputs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    torch.cuda.synchronize()
    return g, outs


def _eager_noise(rng):
    """The program's own eager work between replays (allocations, kernels)."""
    junk = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    junk.copy_(torch.from_numpy(rng.random(1 << 22, dtype=np.float32)))
    del junk


def _same(a, b, what):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b), what


def _replay_rounds(label, static, fill, run, seed):
    """static: dict of input tensors the graph reads; fill(rng) -> dict of new
    host inputs (same shapes); run() -> tuple of outputs."""
    g, outs = _capture(run)
    rng = np.random.default_rng(seed)
    for r in range(REPLAYS):
        new = fill(rng)
        for name, t in static.items():
            t.copy_(new[name])
        torch.cuda.synchronize()
        want = tuple(o.clone() for o in run())   # eager, same inputs
        torch.cuda.synchronize()
        _eager_noise(rng)
        say(f"[graphs] {label}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, want)):
            _same(a, b, f"{label}: replay {r}, output {i}")


def _bf16(rng, shape, scale=1.0):
    return to_gpu_bf16(gen.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * scale))


def test_prefill_step_mask_build_and_forward():
    B, H, S, D, topk = 2, 16, 4096, 64, 16
    nb = S // 64
    rng = np.random.default_rng(1)
    static = {"q": _bf16(rng, (B, H, S, D)), "k": _bf16(rng, (B, H, S, D)),
              "v": _bf16(rng, (B, H, S, D)),
              "scores": to_gpu(rng.standard_normal((B, H, nb, nb), dtype=np.float32))}

    def fill(r):
        return {"q": _bf16(r, (B, H, S, D)), "k": _bf16(r, (B, H, S, D)), "v": _bf16(r, (B, H, S, D)),
                "scores": to_gpu(r.standard_normal((B, H, nb, nb), dtype=np.float32))}

    def run():
        m = bsa.bsattn_build_mask_topk(static["scores"], topk, False, True)
        return m, bsa.bsattn_fwd(static["q"], static["k"], static["v"], m, True)

    _replay_rounds("prefill step", static, fill, run, 2)


@pytest.mark.parametrize("D", [64, 128])
def test_long_row_split_forward_and_merge(D):
    B, H, S = 1, 2, 8400
    nb = -(-S // 64)
    rng = np.random.default_rng(3 + D)

    def mask(r):
        m = (r.random((B, H, nb, nb)) < 0.2).astype(np.uint8)
        m[..., nb - 3:, :] = 1                      # long rows: split in two and merged
        m[..., np.arange(nb), np.arange(nb)] = 1
        return to_gpu(m)

    static = {"q": _bf16(rng, (B, H, S, D)), "k": _bf16(rng, (B, H, S, D)),
              "v": _bf16(rng, (B, H, S, D)), "m": mask(rng)}

    def fill(r):
        return {"q": _bf16(r, (B, H, S, D)), "k": _bf16(r, (B, H, S, D)), "v": _bf16(r, (B, H, S, D)),
                "m": mask(r)}

    ws = torch.empty(bsa.bsattn_fwd_workspace_bytes(B, H, S, D), dtype=torch.uint8, device="cuda")

    def run():
        return (bsa.bsattn_fwd(static["q"], static["k"], static["v"], static["m"], True,
                               workspace=ws),)

    _replay_rounds(f"long-row split D={D}", static, fill, run, 4 + D)


def test_fused_threshold_with_split():
    B, H, S, D = 1, 2, 8400, 64
    nb = -(-S // 64)
    rng = np.random.default_rng(5)

    def scores(r):
        x = r.random((B, H, nb, nb), dtype=np.float32)
        x[..., nb - 2:, :] = 1.0                    # dense last rows: split
        return to_gpu(x)

    static = {"q": _bf16(rng, (B, H, S, D)), "k": _bf16(rng, (B, H, S, D)),
              "v": _bf16(rng, (B, H, S, D)), "s": scores(rng)}

    def fill(r):
        return {"q": _bf16(r, (B, H, S, D)), "k": _bf16(r, (B, H, S, D)), "v": _bf16(r, (B, H, S, D)),
                "s": scores(r)}

    def run():
        return bsa.bsattn_fwd_threshold(static["q"], static["k"], static["v"], static["s"], 0.9,
                                        False, True, True, write_mask=True)

    _replay_rounds("fused threshold", static, fill, run, 6)


def _decode_static(rng, B, Hq, Hkv, D, lens, max_sel):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])

    def idx(r):
        out = np.full((B, Hkv, max_sel), -1, np.int32)
        for b, L in enumerate(lens):
            nbb = -(-int(L) // 64)
            n = min(max_sel, nbb)
            for h in range(Hkv):
                out[b, h, :n] = r.choice(nbb, n, replace=False)
        return to_gpu(out)

    def fill(r):
        return {"q": _bf16(r, (B, Hq, D)), "k": _bf16(r, (T, Hkv, D)), "v": _bf16(r, (T, Hkv, D)),
                "idx": idx(r)}

    static = fill(rng)
    static["cu"] = to_gpu(cu)
    return static, fill


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_split_and_merge(noalloc):
    B, Hq, Hkv, D = 4, 32, 8, 128
    lens = np.array([4096, 700, 12000, 65])
    rng = np.random.default_rng(7 + noalloc)
    static, fill0 = _decode_static(rng, B, Hq, Hkv, D, lens, 48)

    def fill(r):
        d = fill0(r)
        d["cu"] = static["cu"]
        return d

    call = bsa.bsattn_decode_gqa_noalloc if noalloc else bsa.bsattn_decode_gqa

    def run():
        return (call(static["q"], static["k"], static["v"], static["cu"], static["idx"],
                     num_splits=4),)

    _replay_rounds(f"decode noalloc={noalloc}", static, fill, run, 8)


def test_xattn_estimate():
    B, H, S, D, stride = 1, 2, 2048, 128, 8
    rng = np.random.default_rng(9)

    def fill(r):
        return {"q": _bf16(r, (B, H, S, D)), "k": _bf16(r, (B, H, S, D))}

    static = fill(rng)

    def run():
        return bsa.bsattn_xattn_estimate(static["q"], static["k"], stride, 1.0, 0.9, True, True,
                                         True, write_sums=True)

    _replay_rounds("xattn estimate", static, fill, run, 10)
